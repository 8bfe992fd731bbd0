"""C-ABI checks that need no GPU: the library loads, exports every function include/*.h declares,
the size/layout helpers agree with the documented layouts, and argument validation returns the
documented status before anything is launched (no compute call is made)."""
import ctypes as C
import glob
import os
import re

import pytest

from bit_attention_amd import binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[\w]+\s*\*?\s+(sage_\w+)\s*\(", txt, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"sage_fp4_quant", "sage_fp4_attn_fwd"} <= names
    L = bnd.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    assert set(bnd.EXPORTS) == names


def test_constants_and_slot_order():
    assert bnd.sage_fp4_kv_tile() == 128
    assert bnd.sage_fp4_version() >= 300
    order = [bnd.sage_fp4_slot_token(s) for s in range(128)]
    assert sorted(order) == list(range(128))
    assert order[:8] == [0, 1, 2, 3, 16, 17, 18, 19]
    assert order[32] == 4 and bnd.sage_fp4_slot_token(128) == -1 and bnd.sage_fp4_slot_token(-1) == -1


@pytest.mark.parametrize("fmt,blk", [(0, 16), (1, 32), (2, 32)])
def test_size_helpers(fmt, blk):
    B, H, N, D = 2, 3, 300, 128
    assert bnd.sage_fp4_codes_bytes(0, fmt, B, H, N, D) == B * H * N * D // 2
    assert bnd.sage_fp4_scales_bytes(1, fmt, B, H, N, D) == B * H * N * D // blk
    assert bnd.sage_fp4_codes_bytes(2, fmt, B, H, N, D) == B * H * D * 384 // (1 if fmt == 2 else 2)
    assert bnd.sage_fp4_scales_bytes(2, fmt, B, H, N, D) == B * H * D * 384 // blk
    assert bnd.sage_fp4_codes_bytes(0, fmt, B, H, N, 96) == 0
    assert bnd.sage_fp4_codes_bytes(5, fmt, B, H, N, D) == 0


FAKE = C.c_void_p(0x10000)  # never dereferenced: validation fails before any launch
MIS = C.c_void_p(0x10008)


def test_quant_validation():
    q = bnd.sage_fp4_quant
    assert q(3, 0, FAKE, 1, 1, 16, 64, FAKE, FAKE, None) == -5
    assert q(0, 3, FAKE, 1, 1, 16, 64, FAKE, FAKE, None) == -5
    assert q(2, 2, MIS, 1, 1, 16, 64, FAKE, FAKE, None) == -4
    assert q(0, 0, None, 1, 1, 16, 64, FAKE, FAKE, None) == -1
    assert q(0, 0, FAKE, 1, 1, 16, 64, None, FAKE, None) == -1
    assert q(0, 0, FAKE, 1, 1, 16, 96, FAKE, FAKE, None) == -3
    assert q(0, 0, FAKE, 0, 1, 16, 64, FAKE, FAKE, None) == -2
    assert q(0, 0, FAKE, 1, 1, 0, 64, FAKE, FAKE, None) == -2
    assert q(0, 0, FAKE, 1, 1, (1 << 20) + 1, 64, FAKE, FAKE, None) == -2
    assert q(0, 0, MIS, 1, 1, 16, 64, FAKE, FAKE, None) == -4
    # B*H*N*D < 2^36: B*H = 1024, N = 2^20, D = 64 is exactly 2^36
    assert q(0, 0, FAKE, 1, 1024, 1 << 20, 64, FAKE, FAKE, None) == -2
    assert q(2, 1, FAKE, 2, 512, 1 << 20, 64, FAKE, FAKE, None) == -2


def test_element_limit_in_size_queries():
    """The size queries accept the largest shape under 2^36 elements and reject 2^36."""
    assert bnd.sage_fp4_codes_bytes(0, 0, 1, 1023, 1 << 20, 64) == 1023 * (1 << 20) * 32
    assert bnd.sage_fp4_codes_bytes(0, 0, 1, 1024, 1 << 20, 64) == 0
    assert bnd.sage_fp4_scales_bytes(2, 1, 1, 511, 1 << 20, 128) == 511 * 128 * ((1 << 20) // 32)
    assert bnd.sage_fp4_scales_bytes(2, 1, 1, 512, 1 << 20, 128) == 0


def test_attn_validation():
    a = bnd.sage_fp4_attn_fwd
    ok = [FAKE] * 6
    assert a(3, *ok, 1, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -5
    assert a(2, *ok, 1, 1, 16, 96, 0, 0.0, FAKE, 1, None) == -3
    assert a(0, *ok, 1, 1, 16, 64, 0, 0.0, FAKE, 7, None) == -5
    assert a(0, *ok[:5], None, 1, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -1
    assert a(0, *ok, 1, 1, 16, 64, 0, 0.0, None, 1, None) == -1
    assert a(0, *ok, 1, 1, 16, 32, 0, 0.0, FAKE, 1, None) == -3
    assert a(0, *ok, 1, -1, 16, 64, 0, 0.0, FAKE, 1, None) == -2
    assert a(0, *ok[:2], MIS, *ok[3:], 1, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -4
    assert a(0, *ok, 1, 1, 16, 64, 0, 0.0, MIS, 1, None) == -4
    for s in (0, -1, -2, -3, -4, -5, -6, 99):
        assert isinstance(bnd.status_string(s), str) and bnd.status_string(s)


def test_attn_direct_p_validation():
    a = bnd.sage_fp4_attn_fwd_direct_p
    ok = [FAKE] * 6
    assert a(*ok, 1, 1, 16, 64, 0, 0.0, FAKE, 7, None) == -5
    assert a(*ok[:5], None, 1, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -1
    assert a(None, *ok[1:], 1, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -1
    assert a(*ok, 1, 1, 16, 64, 0, 0.0, None, 0, None) == -1
    assert a(*ok, 1, 1, 16, 96, 1, 0.0, FAKE, 1, None) == -3
    assert a(*ok, 1, 1, 0, 64, 0, 0.0, FAKE, 1, None) == -2
    assert a(*ok, 70000, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -2
    assert a(*ok[:4], MIS, ok[5], 1, 1, 16, 64, 0, 0.0, FAKE, 1, None) == -4
    assert a(*ok, 1, 1, 16, 128, 1, 0.0, MIS, 0, None) == -4


def test_library_does_not_link_the_oracle():
    """The product library and the oracle share no code: no oracle symbol is exported or needed."""
    import subprocess
    out = subprocess.run(["nm", "-D", bnd.LIB_PATH], capture_output=True, text=True).stdout
    assert "orc_" not in out
    deps = subprocess.run(["readelf", "-d", bnd.LIB_PATH], capture_output=True, text=True).stdout
    assert "sage_oracle" not in deps


def test_bwd_workspace_and_validation():
    """Backward entry point: documented workspace size, and every argument check (no launch)."""
    def a256(x):
        return (x + 255) // 256 * 256
    B, H, N, D = 2, 3, 300, 128
    np64, nb = 320, 5
    want = (2 * a256(B * H * N * D * 2) + 3 * a256(B * H * D * np64) + 3 * a256(B * H * D * nb * 4)
            + 2 * a256(B * H * np64 * 4))
    assert bnd.sage_fp4_attn_bwd_workspace_bytes(B, H, N, D) == want
    assert bnd.sage_fp4_attn_bwd_workspace_bytes(B, H, N, 96) == 0
    assert bnd.sage_fp4_attn_bwd_workspace_bytes(1, 1024, 1 << 20, 64) == 0
    need = bnd.sage_fp4_attn_bwd_workspace_bytes(1, 1, 16, 64)
    b = bnd.sage_fp4_attn_bwd
    ok = [FAKE] * 8

    def call(fmt=0, ptrs=ok, D=64, outs=(FAKE, FAKE, FAKE), od=1, ws=FAKE, wsb=need, N=16):
        return b(fmt, *ptrs, 1, 1, N, D, 0, 0.0, *outs, od, ws, wsb, None)

    assert call(wsb=need - 1) == -7
    assert call(ws=None) == -1
    assert call(ptrs=ok[:7] + [None]) == -1
    assert call(outs=(FAKE, None, FAKE)) == -1
    assert call(ptrs=ok[:4] + [MIS] + ok[5:]) == -4
    assert call(outs=(FAKE, FAKE, MIS)) == -4
    assert call(ws=MIS) == -4
    assert call(fmt=3) == -5
    assert call(od=2) == -5
    assert call(D=96) == -3
    assert call(N=0) == -2
    assert bnd.status_string(-7) != bnd.status_string(99)
    st = bnd.sage_fp4_attn_bwd_stage
    assert st(3, 0, *ok, 1, 1, 16, 64, 0, 0.0, FAKE, FAKE, FAKE, 1, FAKE, need, None) == -5
    assert st(-1, 0, *ok, 1, 1, 16, 64, 0, 0.0, FAKE, FAKE, FAKE, 1, FAKE, need, None) == -5
    assert st(1, 0, *ok, 1, 1, 16, 64, 0, 0.0, FAKE, FAKE, FAKE, 1, FAKE, need - 1, None) == -7
    assert st(2, 0, *ok, 1, 1, 16, 64, 0, 0.0, FAKE, None, FAKE, 1, FAKE, need, None) == -1


def test_kv16_bytes_and_validation():
    """Dequantised-K/V entry points: documented buffer size, and every argument check (no launch)."""
    assert bnd.sage_fp4_kv16_bytes(2, 3, 300, 128) == 4 * 2 * 3 * 384 * 128
    assert bnd.sage_fp4_kv16_bytes(1, 1, 1, 64) == 4 * 128 * 64
    assert bnd.sage_fp4_kv16_bytes(2, 3, 300, 96) == 0
    assert bnd.sage_fp4_kv16_bytes(1, 1024, 1 << 20, 64) == 0
    need = bnd.sage_fp4_kv16_bytes(1, 1, 16, 64)
    p = bnd.sage_fp4_kv16_prep
    ok = [FAKE] * 4
    assert p(*ok, 1, 1, 16, 64, FAKE, need - 1, None) == -7
    assert p(*ok, 1, 1, 16, 64, None, need, None) == -1
    assert p(*ok[:3], None, 1, 1, 16, 64, FAKE, need, None) == -1
    assert p(*ok[:2], MIS, ok[3], 1, 1, 16, 64, FAKE, need, None) == -4
    assert p(*ok, 1, 1, 16, 64, MIS, need, None) == -4
    assert p(*ok, 1, 1, 16, 96, FAKE, need, None) == -3
    assert p(*ok, 1, 1, 0, 64, FAKE, need, None) == -2
    a = bnd.sage_fp4_attn_fwd_kv16

    def call(qc=FAKE, qs=FAKE, kv=FAKE, kvb=need, D=64, N=16, out=FAKE, od=1, lse=None):
        return a(qc, qs, kv, kvb, 1, 1, N, D, 0, 0.0, out, od, lse, None)

    assert call(kvb=need - 1) == -7
    assert call(kv=None) == -1
    assert call(qs=None) == -1
    assert call(out=None) == -1
    assert call(od=2) == -5
    assert call(D=96) == -3
    assert call(N=0) == -2
    assert call(qc=MIS) == -4
    assert call(out=MIS) == -4
    assert call(lse=MIS) == -4
    assert call(kv=MIS) == -4
    qk = bnd.sage_fp4_quant_kv16

    def qcall(role=1, x=FAKE, c=FAKE, s=FAKE, kv=FAKE, kvb=need, D=64, N=16):
        return qk(role, x, 1, 1, N, D, c, s, kv, kvb, None)

    assert qcall(role=0) == -5 and qcall(role=3) == -5
    assert qcall(kvb=need - 1) == -7 and qcall(role=2, kvb=need - 1) == -7
    assert qcall(x=None) == -1 and qcall(c=None) == -1 and qcall(s=None) == -1 and qcall(kv=None) == -1
    assert qcall(x=MIS) == -4 and qcall(s=MIS) == -4 and qcall(kv=MIS) == -4
    assert qcall(D=96) == -3 and qcall(N=0) == -2
