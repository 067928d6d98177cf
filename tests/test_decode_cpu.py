"""CPU tests of the decode entry points' host-side validation (no device
work: every call here fails validation before anything is enqueued)."""
import ctypes
import os

import pytest
import torch

import ulysses_sequence_attention_zigzag_amd as usp

pytestmark = pytest.mark.skipif(not os.path.exists(usp.LIB_PATH), reason="libusp.so not built")

FAKE = ctypes.c_void_p(0x10000)


def _split(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ld=None, lh=None, op=FAKE, lp=FAKE, B=2, Lq=1, S=1024, Hq=8, Hkv=2, D=128,
             split=256, scale=0.0, window=0, n_sink=0, cap=0.0, alibi=None)
    a.update(kw)
    st = usp.lib().usp_decode_split_fwd(a["q"], a["k"], a["v"], a["ld"], a["lh"], a["op"], a["lp"], a["B"], a["Lq"],
                                        a["S"], a["Hq"], a["Hkv"], a["D"], a["split"], a["scale"], a["window"],
                                        a["n_sink"], a["cap"], a["alibi"], None)
    return st, usp.lib().usp_last_error().decode()


def test_decode_split_validation():
    assert _split(q=None)[0] == 1
    st, msg = _split(D=96)
    assert st == 2 and "head_dim" in msg
    st, msg = _split(Hq=6, Hkv=4)
    assert st == 1 and "multiple" in msg
    # 32 queries per KV head is the limit (this call still fails later, on split_keys)
    st, msg = _split(Hq=32, Hkv=1, split=100)
    assert st == 1 and "split_keys" in msg
    st, msg = _split(Hq=32, Hkv=1, Lq=2)
    assert st == 2 and "32 queries" in msg
    st, msg = _split(split=100)
    assert st == 1 and "split_keys" in msg
    st, msg = _split(Lq=20, S=16, Hq=2, Hkv=2)
    assert st == 1 and "Lq" in msg
    st, msg = _split(window=-1)
    assert st == 1 and "window" in msg
    lens = torch.tensor([1024, 0], dtype=torch.int32)
    st, msg = _split(ld=FAKE, lh=ctypes.c_void_p(lens.data_ptr()))
    assert st == 1 and "kv_lens[1]" in msg
    st, msg = _split(ld=None, lh=ctypes.c_void_p(lens.data_ptr()))
    assert st == 1 and "both" in msg
    st, msg = _split(scale=float("inf"))
    assert st == 1 and "finite" in msg
    st, msg = _split(cap=-1.0)
    assert st == 1 and "softcap" in msg
    st, msg = _split(S=(1 << 22) + 32, Hkv=1, D=64, alibi=FAKE)
    assert st == 2 and "ALiBi" in msg


def test_decode_merge_validation():
    L = usp.lib()
    st = L.usp_decode_merge(FAKE, FAKE, 0, 1, 1, 8, 128, FAKE, 1, FAKE, None)
    assert st == 1 and "sizes" in L.usp_last_error().decode()
    st = L.usp_decode_merge(FAKE, FAKE, 4, 1, 1, 8, 80, FAKE, 1, FAKE, None)
    assert st == 2
    st = L.usp_decode_merge(None, FAKE, 4, 1, 1, 8, 128, FAKE, 1, FAKE, None)
    assert st == 1
    st = L.usp_decode_merge(FAKE, FAKE, 4, 1, 1, 8, 128, FAKE, 5, FAKE, None)
    assert st == 1 and "dtype" in L.usp_last_error().decode()
