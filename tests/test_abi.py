"""C-ABI contract checks that need no GPU: exports, validation codes, error text, pair counts."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import sinks_ts_mha_amd as tm
from sinks_ts_mha_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ts_mha.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ts_mha_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["ts_mha_decode_with_kvcache", "ts_mha_decode_with_kvcache_noalloc",
                                    "ts_mha_decode_workspace_size", "ts_mha_prefill",
                                    "ts_mha_prefill_with_kvcache", "ts_mha_strerror",
                                    "ts_mha_unmasked_pairs"]


def test_library_exports_every_declared_symbol():
    lib = tm.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ts_mha_\w+)$", nm, flags=re.M))
    assert set(declared_functions()) <= exported


def test_error_codes_match_header():
    text = open(HEADER).read()
    codes = {name: int(val) for name, val in
             re.findall(r"#define (TS_MHA_ERR_\w+) \((-\d+)\)", text)}
    assert codes == {v: k for k, v in _binding.ERROR_NAMES.items()}


FAKE = 0x10000  # aligned, never dereferenced: every case below is rejected on the host


def call(q=FAKE, k=FAKE, v=FAKE, sinks=None, cu=FAKE, hq=64, hkv=8, d=64, window=0,
         scale=0.125, out=FAKE * 2, n_seqs=4, max_seqlen=2048, stream=None):
    return tm.lib().ts_mha_prefill(q, k, v, sinks, cu, hq, hkv, d, window, scale, out, n_seqs,
                                   max_seqlen, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(cu=None), -1),
    (dict(out=None), -1),
    (dict(hq=0), -2), (dict(hkv=0), -2), (dict(hq=-8), -2), (dict(hq=12, hkv=8), -2),
    (dict(n_seqs=-1), -2), (dict(max_seqlen=-5), -2),
    (dict(max_seqlen=2**31 - 1, n_seqs=2**20), -2),
    # one sequence's q rows beyond 2^31 - 1 bytes: (262000 + 256) * 64 heads * 128 B
    (dict(max_seqlen=262000, n_seqs=1), -2),
    # its k/v rows beyond 2^31 - 1 bytes with few q heads: (2**21 + 64) * 8 * 128 B
    (dict(max_seqlen=2**21, hq=8, hkv=8, n_seqs=1), -2),
    # at head_dim 128: (131100 + 128) * 64 heads * 256 B
    (dict(d=128, max_seqlen=131100, n_seqs=1), -2),
    # one token past the largest accepted sequence (see test_validation_precedes_device_check)
    (dict(max_seqlen=261888, n_seqs=1), -2), (dict(d=128, max_seqlen=130944, n_seqs=1), -2),
    (dict(d=256), -3), (dict(d=96), -3), (dict(d=32), -3), (dict(hq=24, hkv=8), -3),
    (dict(hq=64, hkv=2), -3), (dict(d=128, hq=64, hkv=2), -3),
    (dict(scale=0.0), -4), (dict(scale=-0.1), -4), (dict(scale=float("nan")), -4),
    (dict(scale=float("inf")), -4),
    (dict(q=FAKE + 8), -5), (dict(k=FAKE + 2), -5), (dict(v=FAKE + 4), -5),
    (dict(out=FAKE + 12), -5), (dict(sinks=FAKE + 2), -5), (dict(cu=FAKE + 1), -5),
])
def test_host_validation_codes(kw, code):
    assert call(**kw) == code


def test_validation_precedes_device_check():
    # With valid arguments the only remaining failure on a GPU-less host is "no device";
    # on a GPU host this test is skipped because the call would really launch.
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call() == -6
    assert call(window=128, sinks=FAKE) == -6
    assert call(n_seqs=0, max_seqlen=0) == -6
    assert call(max_seqlen=261000, n_seqs=1) == -6  # just inside the q-row limit
    # the largest accepted sequences: (L + 256) * 64 heads * 128 B and (L + 128) * 64 * 256 B
    # within 2^31 - 1 (the GPU parity suite runs both)
    assert call(max_seqlen=261887, n_seqs=1) == -6 and call(d=128, max_seqlen=130943, n_seqs=1) == -6
    assert call(d=128) == -6 and call(d=128, window=128, sinks=FAKE) == -6
    assert call(d=128, max_seqlen=130000, n_seqs=1) == -6  # inside the head_dim 128 limit


def test_strerror_texts():
    for code in list(_binding.ERROR_NAMES) + [0]:
        text = tm.ts_mha_strerror(code)
        assert text and text != "unknown error"
    assert tm.ts_mha_strerror(12345) == "unknown error"
    assert "HIP launch failed" in tm.ts_mha_strerror(-8)


def brute_pairs(seqlens, window):
    n = 0
    for L in seqlens:
        for i in range(L):
            for j in range(i + 1):
                if window <= 0 or i - j < window:
                    n += 1
    return n


@pytest.mark.parametrize("seqlens,window", [([5], 0), ([5], 2), ([0, 3, 7], 3), ([1, 1], 1),
                                            ([10, 20, 30], 0), ([10, 20, 30], 15),
                                            ([64, 65], 64), ([33], 100), ([], 0)])
def test_unmasked_pairs_brute_force(seqlens, window):
    cu = [0]
    for L in seqlens:
        cu.append(cu[-1] + L)
    assert tm.ts_mha_unmasked_pairs(cu, window) == brute_pairs(seqlens, window)


def test_unmasked_pairs_workloads():
    from sinks_ts_mha_amd.workloads import WORKLOADS
    expect = {"tiny_1x128_gqa4": 8256, "gptoss_full_4x2048": 8392704,
              "gptoss_window128_4x2048": 1016064, "varlen16_window128": 9900928,
              "long_1x32768": 536887296}
    for name, n in expect.items():
        wl = WORKLOADS[name]
        assert tm.ts_mha_unmasked_pairs(wl.cu_seqlens(), wl.window) == n


def test_unmasked_pairs_rejects_bad_input():
    L = tm.lib()
    assert L.ts_mha_unmasked_pairs(None, 1, 0) == -1
    arr = (ctypes.c_int32 * 3)(0, 5, 3)
    assert L.ts_mha_unmasked_pairs(arr, 2, 0) == -1
    assert L.ts_mha_unmasked_pairs(arr, -1, 0) == -1


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        tm.ts_mha_prefill(q, q[:, :1].contiguous(), q[:, :1].contiguous(), None, cu, max_seqlen=4)
    with pytest.raises(TypeError):
        tm.ts_mha_prefill(q.float(), q, q, None, cu, max_seqlen=4)


# ---- decode against a paged KV cache

def dcall(q=FAKE, kc=FAKE, vc=FAKE, sinks=None, lens=FAKE, table=FAKE, hq=64, hkv=8, d=64,
          window=0, scale=0.125, out=FAKE * 2, n_seqs=64, n_pages=40000, page=16, pps=512,
          max_k=8192, ws=FAKE * 4, ws_bytes=1 << 30, stream=None):
    return tm.lib().ts_mha_decode_with_kvcache(q, kc, vc, sinks, lens, table, hq, hkv, d, window,
                                               scale, out, n_seqs, n_pages, page, pps, max_k, ws,
                                               ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(vc=None), -1), (dict(lens=None), -1),
    (dict(table=None), -1), (dict(out=None), -1),
    (dict(hq=0), -2), (dict(hq=12, hkv=8), -2), (dict(n_seqs=-1), -2), (dict(max_k=-1), -2),
    (dict(n_pages=0), -2), (dict(pps=0), -2), (dict(page=8), -2), (dict(page=24), -2),
    (dict(page=0), -2), (dict(max_k=512 * 16 + 1), -2), (dict(page=1 << 20, hkv=64, hq=64), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(hq=64, hkv=2), -3),
    (dict(scale=0.0), -4), (dict(scale=float("nan")), -4),
    (dict(q=FAKE + 8), -5), (dict(kc=FAKE + 4), -5), (dict(out=FAKE + 2), -5),
    (dict(table=FAKE + 2), -5), (dict(ws=FAKE + 64), -5),
    (dict(ws=None, n_seqs=1), -10), (dict(ws_bytes=1024, n_seqs=1), -10),
])
def test_decode_host_validation_codes(kw, code):
    assert dcall(**kw) == code


def test_decode_workspace_size():
    ws = tm.ts_mha_decode_workspace_size
    # many sequences with a short context: one chunk per sequence, no workspace
    assert ws(256, 64, 8, 64, 0, 2048) == 0
    assert ws(64, 64, 8, 64, 128, 8192) >= 0
    # one long sequence is split into chunks whose partial rows need a workspace
    big = ws(1, 64, 8, 64, 0, 65536)
    assert big > 0 and big % 4 == 0
    assert ws(1, 64, 8, 64, 0, 65536) == big  # a function of its arguments only
    assert ws(0, 64, 8, 64, 0, 0) == 0
    # head_dim 128 with 2 KV heads (the same work-groups and split as head_dim 64): twice the
    # partial output per row
    d64, d128 = ws(1, 16, 2, 64, 0, 65536), ws(1, 16, 2, 128, 0, 65536)
    assert d64 > 0 and d128 > d64 and (d128 - d64) % (16 * 64 * 4) == 0
    with pytest.raises(tm.TsMhaError):
        ws(1, 64, 8, 96, 0, 1024)
    with pytest.raises(tm.TsMhaError):
        ws(1, 12, 8, 64, 0, 1024)


def test_decode_validation_precedes_device_check():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert dcall() == -6
    assert dcall(n_seqs=0) == -6
    assert dcall(n_seqs=1, max_k=65536, pps=4096, ws_bytes=1 << 30) == -6
    assert dcall(ws=None, max_k=2048, n_seqs=256) == -6  # no workspace needed there
    assert dcall(d=128) == -6 and dcall(d=128, n_seqs=1, max_k=65536, pps=4096, ws_bytes=1 << 30) == -6


# ---- prefill of new rows against a paged KV cache

def pcall(q=FAKE, kc=FAKE, vc=FAKE, sinks=None, cu=FAKE, lens=FAKE, table=FAKE, hq=64, hkv=8, d=64,
          window=0, scale=0.125, out=FAKE * 2, n_seqs=4, n_pages=4000, page=16, pps=512,
          max_q=2048, max_k=8192, stream=None):
    return tm.lib().ts_mha_prefill_with_kvcache(q, kc, vc, sinks, cu, lens, table, hq, hkv, d, window,
                                                scale, out, n_seqs, n_pages, page, pps, max_q, max_k,
                                                stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(vc=None), -1), (dict(cu=None), -1),
    (dict(lens=None), -1), (dict(table=None), -1), (dict(out=None), -1),
    (dict(hq=0), -2), (dict(hq=12, hkv=8), -2), (dict(n_seqs=-1), -2), (dict(max_k=-1), -2),
    (dict(max_q=-1), -2), (dict(max_q=8193), -2), (dict(page=8), -2), (dict(n_pages=0), -2),
    (dict(pps=0), -2), (dict(max_k=512 * 16 + 1), -2),
    # one sequence's q rows beyond 2^31 - 1 bytes
    (dict(max_q=262000, max_k=262000, pps=16384, n_seqs=1), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(hq=64, hkv=2), -3),
    (dict(scale=0.0), -4), (dict(scale=float("inf")), -4),
    (dict(q=FAKE + 8), -5), (dict(vc=FAKE + 4), -5), (dict(out=FAKE + 2), -5), (dict(cu=FAKE + 2), -5),
    (dict(lens=FAKE + 1), -5),
])
def test_prefill_kvcache_host_validation_codes(kw, code):
    assert pcall(**kw) == code


def test_prefill_kvcache_validation_precedes_device_check():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert pcall() == -6
    assert pcall(n_seqs=0, max_q=0, max_k=0) == -6
    assert pcall(window=128, sinks=FAKE) == -6
    assert pcall(d=128) == -6 and pcall(d=128, window=128, page=64) == -6
