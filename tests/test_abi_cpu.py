"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, rejects bad arguments before touching the device, and its
host RoPE table matches the oracle's bit for bit."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from head_latent_attention_05_amd import binding as B
from head_latent_attention_05_amd import synth
from oracle import mla_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
FAKE = 0x100000  # aligned, non-null; never dereferenced on the early-return paths


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings():
    lib = B.load()
    for code in range(5):
        s = lib.mla_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.mla_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("d_rope,max_pos", [(64, 40000), (16, 300)])
def test_rope_table_matches_oracle_bitwise(d_rope, max_pos):
    cos, sin = B.rope_table(max_pos, d_rope)
    oc, os_ = O.rope_table_f32(max_pos, d_rope)
    np.testing.assert_array_equal(cos.view(np.uint32), oc.view(np.uint32))
    np.testing.assert_array_equal(sin.view(np.uint32), os_.view(np.uint32))


def test_rope_table_rejects_bad_args():
    lib = B.load()
    buf = np.zeros(64, np.float32)
    assert lib.mla_rope_table(None, buf.ctypes.data, 4, 16, 1e4) == 1
    assert lib.mla_rope_table(buf.ctypes.data, buf.ctypes.data, 4, 15, 1e4) == 1
    assert lib.mla_rope_table(buf.ctypes.data, buf.ctypes.data, 0, 16, 1e4) == 1


def _cfg(dims=synth.V3, **kw):
    c = B.MlaConfig.from_dims(dims)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_validation():
    lib = B.load()
    P = ctypes.c_void_p
    # unsupported: bf16 with non-V3 dims; fp32 with a latent width not built
    for c in (_cfg(num_heads=64), _cfg(synth.TINY, d_latent=96), _cfg(block_size=32)):
        assert lib.mla_absorb_q(ctypes.byref(c), 1, P(FAKE), P(FAKE), P(FAKE), None) == 2
    # invalid: odd rope width, bad scale, bad dtype, null config
    for c in (_cfg(d_rope=63), _cfg(softmax_scale=0.0), _cfg(dtype=7)):
        assert lib.mla_absorb_q(ctypes.byref(c), 1, P(FAKE), P(FAKE), P(FAKE), None) == 1
    assert lib.mla_absorb_q(None, 1, P(FAKE), P(FAKE), P(FAKE), None) == 1


def test_projection_argument_checks():
    lib = B.load()
    c = _cfg()
    P = ctypes.c_void_p
    assert lib.mla_absorb_q(ctypes.byref(c), 0, None, None, None, None) == 0   # T=0 no-op
    assert lib.mla_absorb_q(ctypes.byref(c), -1, P(FAKE), P(FAKE), P(FAKE), None) == 1
    assert lib.mla_absorb_q(ctypes.byref(c), 1, None, P(FAKE), P(FAKE), None) == 1
    assert lib.mla_absorb_q(ctypes.byref(c), 1, P(FAKE + 2), P(FAKE), P(FAKE), None) == 1
    assert lib.mla_out_proj(ctypes.byref(c), 0, None, None, None, None) == 0
    assert lib.mla_out_proj(ctypes.byref(c), 2, P(FAKE), P(FAKE + 8), P(FAKE), None) == 1
    # token count above the limit the header documents
    big = int(re.search(r"#define MLA_MAX_PROJ_TOKENS (\d+)", open(HEADER).read()).group(1)) + 1
    assert lib.mla_absorb_q(ctypes.byref(c), big, P(FAKE), P(FAKE), P(FAKE), None) == 1
    assert lib.mla_out_proj(ctypes.byref(c), big, P(FAKE), P(FAKE), P(FAKE), None) == 1


def test_append_argument_checks():
    lib = B.load()
    c = _cfg()
    P = ctypes.c_void_p
    args = [P(FAKE)] * 7
    ok_tail = [3, 4, 10, P(FAKE), P(FAKE), 64, P(FAKE), None, None, None]
    # q_pe given without q_lat
    assert lib.mla_append_cache(ctypes.byref(c), 2, *args[:2], P(FAKE), *args[3:6],
                                3, 4, 10, P(FAKE), P(FAKE), 64, P(FAKE), None, None, None) == 1
    # missing pool / table / rope
    assert lib.mla_append_cache(ctypes.byref(c), 2, *args[:2], None, *args[3:6], 3, 4, 10,
                                P(FAKE), P(FAKE), 64, None, None, None, None) == 1
    assert lib.mla_append_cache(ctypes.byref(c), 2, *args[:2], None, *args[3:6], 3, 4, 10,
                                None, P(FAKE), 64, P(FAKE), None, None, None) == 1
    # bad sizes
    assert lib.mla_append_cache(ctypes.byref(c), 2, *args[:2], None, *args[3:6], 0, 4, 10,
                                P(FAKE), P(FAKE), 64, P(FAKE), None, None, None) == 1
    assert lib.mla_append_cache(ctypes.byref(c), 0, None, None, None, None, None, None, 0, 0, 0,
                                None, None, 0, None, None, None, None) == 0


def _ws(c, qs, kl, causal=0, G=0):
    lib = B.load()
    qs = np.asarray(qs, np.int32)
    kl = np.asarray(kl, np.int32)
    out = ctypes.c_size_t(0)
    st = lib.mla_decode_workspace_size(ctypes.byref(c), len(kl), qs.ctypes.data, kl.ctypes.data,
                                       causal, G, ctypes.byref(out))
    return st, out.value


def test_workspace_size_and_length_checks():
    c = _cfg()
    st, n = _ws(c, [0, 1, 2], [100, 5000], G=1)
    assert st == 0 and n == 0                       # one workgroup: no partials
    st, n = _ws(c, [0, 1, 2], [100, 5000], G=16)
    assert st == 0
    lse = 2 * 16 * 128 * 4
    assert n == ((lse + 255) // 256) * 256 + 2 * 16 * 128 * 512 * 2
    # G is clamped to the number of units (blocks over all query tokens)
    st, n_big = _ws(c, [0, 1], [64], G=50)
    assert st == 0 and n_big == 0                   # one unit -> one workgroup
    assert _ws(c, [1, 2], [10], G=4)[0] == 1        # q_start must start at 0
    assert _ws(c, [0, 3], [2], G=4)[0] == 1         # more queries than kv rows
    assert _ws(c, [0, 1], [0], G=4)[0] == 1         # empty sequence
    assert _ws(c, [0, 2, 1], [5, 5], G=4)[0] == 1   # q_start decreasing
    assert _ws(c, [0, 512, 1024], [16384, 16384], causal=1, G=4)[0] == 0


def test_decode_rejects_small_workspace_before_launch():
    lib = B.load()
    c = _cfg()
    P = ctypes.c_void_p
    qs = np.array([0, 1], np.int32)
    kl = np.array([4096], np.int32)
    st = lib.mla_decode(ctypes.byref(c), 1, P(FAKE), P(FAKE), qs.ctypes.data, kl.ctypes.data,
                        P(FAKE), 64, 100, P(FAKE), P(FAKE), 0, 8, P(FAKE), 16, P(FAKE), None,
                        None)
    assert st == 3
    # block table too narrow for the longest sequence
    st = lib.mla_decode(ctypes.byref(c), 1, P(FAKE), P(FAKE), qs.ctypes.data, kl.ctypes.data,
                        P(FAKE), 63, 100, P(FAKE), P(FAKE), 0, 8, P(FAKE), 1 << 30, P(FAKE),
                        None, None)
    assert st == 1
    # block table with 2^31 entries or more: its device indices are 32-bit
    qs2 = np.array([0, 1, 2], np.int32)
    kl2 = np.array([4096, 4096], np.int32)
    st = lib.mla_decode(ctypes.byref(c), 2, P(FAKE), P(FAKE), qs2.ctypes.data, kl2.ctypes.data,
                        P(FAKE), 1 << 30, 100, P(FAKE), P(FAKE), 0, 8, P(FAKE), 1 << 30,
                        P(FAKE), None, None)
    assert st == 2
