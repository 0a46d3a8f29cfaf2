"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/gdn.h and include/gqa.h, and rejects bad arguments on the host before any HIP
call (every call here fails validation, so nothing is ever enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from hybrid_linear_attention_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(gdn.LIB_PATH),
                                reason="libgdn.so not built (run __graft_entry__.build())")

FULL = gdn.GdnDimsC(16, 48, 128, 128, 4)
FAKE = 0x10000  # 64 KiB-aligned non-null address; never dereferenced (validation fails first)


def declared_functions():
    names = set()
    for h in ("gdn.h", "gqa.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b((?:gdn|gqa)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    lib = gdn.lib()
    names = declared_functions()
    assert "gdn_decode_step" in names and "gdn_prefill_varlen" in names and "gqa_decode_paged" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) <= set(gdn._SIGS), "binding is missing a declared entry point"


def test_status_strings_and_version():
    lib = gdn.lib()
    for code in range(9):
        assert lib.gdn_status_string(code).decode().startswith(gdn.STATUS[code])
    assert b"gfx950" in lib.gdn_version()


def dims(*v):
    return gdn.GdnDimsC(*v)


def decode_call(d, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, act=0, a=FAKE, b=FAKE, gdt=1, gld=48, state=FAKE,
                slots=FAKE, R=4, nslots=8, o=FAKE, odt=0)
    args.update(kw)
    return gdn.lib().gdn_decode_step(
        None if d is None else ctypes.byref(d), args["q"], args["k"], args["v"], args["act"],
        args["a"], args["b"], args["gdt"], args["gld"], args["state"], args["slots"], args["R"],
        args["nslots"], args["o"], args["odt"], None)


@pytest.mark.parametrize("bad,status", [
    (None, 1),
    ((16, 48, 128, 128, 3), 2),     # conv taps
    ((16, 40, 128, 128, 4), 2),     # Hv % Hk
    ((16, 48, 128, 64, 4), 2),      # dk != dv
    ((16, 48, 96, 96, 4), 2),       # unsupported head dim
    ((0, 48, 128, 128, 4), 2),
])
def test_decode_rejects_bad_dims(bad, status):
    d = None if bad is None else dims(*bad)
    assert decode_call(d) == status


def test_decode_rejects_bad_args():
    assert decode_call(FULL, act=2) == 3
    assert decode_call(FULL, R=-1) == 4
    assert decode_call(FULL, R=9, nslots=8) == 4
    assert decode_call(FULL, gld=47) == 4
    assert decode_call(FULL, q=None) == 1
    assert decode_call(FULL, state=None) == 1
    assert decode_call(FULL, state=FAKE + 4) == 6
    assert decode_call(FULL, q=FAKE + 8, act=0) == 6  # fp32 q needs 16 bytes
    assert decode_call(FULL, R=0, q=None) == 0        # nothing to do, nothing enqueued


def test_prefill_and_conv_reject_bad_args():
    lib = gdn.lib()
    P = FAKE

    def prefill(**kw):
        a = dict(T=10, R=2, nslots=4, qsl=P, ws=None, wsb=0, gld=48, act=1)
        a.update(kw)
        return lib.gdn_prefill_varlen(ctypes.byref(FULL), P, P, P, a["act"], P, P, 1, a["gld"], P,
                                      a["qsl"], P, None, a["R"], a["T"], a["nslots"], P, 0, a["ws"],
                                      a["wsb"], None)
    assert prefill(T=10, R=0) == 4
    assert prefill(R=5) == 4
    assert prefill(qsl=None) == 1
    assert prefill(gld=10) == 4
    assert prefill(act=7) == 3
    assert prefill(T=0) == 0

    def conv(**kw):
        a = dict(x=P, xdt=1, xld=10240, pdt=1, T=16, R=2, nslots=2, eps=1e-6, out=P)
        a.update(kw)
        return lib.gdn_conv1d_update(ctypes.byref(FULL), a["x"], a["xdt"], a["xld"], P, 1, P,
                                     a["pdt"], P, P, None, a["R"], a["T"], a["nslots"], a["eps"],
                                     a["out"], P, P, 0, None)
    assert conv(pdt=0) == 3               # pool dtype must equal x dtype
    assert conv(xld=10000) == 4           # row stride shorter than Cqkv
    assert conv(R=3) == 4                 # more requests than slots
    assert conv(x=None) == 1
    assert conv(x=P + 2) == 6             # bf16 pairs need 4-byte alignment
    assert conv(xld=10241) == 6           # odd row stride breaks pair alignment
    assert conv(eps=float("nan")) == 4
    assert conv(T=0) == 0


def test_norm_and_gemm_reject_bad_args():
    lib = gdn.lib()
    P = FAKE
    assert lib.gdn_gated_norm(ctypes.byref(FULL), P, 0, P, 1, 6000, P, 1, 1e-6, 4, P, 1, None) == 4
    assert lib.gdn_gated_norm(ctypes.byref(FULL), P, 0, P, 1, 6144, P, 1, 1e-6, 4, None, 1, None) == 1
    assert lib.gdn_rmsnorm(P, 1, P, 1, 1e-6, 4, 5121, P, 1, None) == 4
    assert lib.gdn_rmsnorm(P, 1, P, 1, 1e-6, 4, 5120, P + 8, 1, None) == 6
    assert lib.gdn_gemm_bf16(P, 64, P, 64, P, 64, 0, None, 0, 10, 64, 60, None) == 4   # K % 8
    assert lib.gdn_gemm_bf16(P, 32, P, 64, P, 64, 0, None, 0, 10, 64, 64, None) == 4   # lda < K
    assert lib.gdn_gemm_bf16(None, 64, P, 64, P, 64, 0, None, 0, 10, 64, 64, None) == 1
    # B is [N, ldb] with ldb >= K (not N): a wide projection, N > K, is valid
    assert lib.gdn_gemm_bf16(P, 64, P, 64, P, 128, 0, None, 0, 0, 128, 64, None) == 0
    assert lib.gdn_gemm_bf16(P, 64, P, 32, P, 128, 0, None, 0, 0, 128, 64, None) == 4
    assert lib.gdn_gemm_bf16(P, 64, P, 64, P, 64, 0, None, 0, 0, 64, 64, None) == 0
    # the workspace variant: same checks, then a 256-byte aligned workspace
    assert lib.gdn_gemm_bf16_ws(P, 64, P, 64, P, 64, 0, None, 0, 10, 64, 60, None, 0, None) == 4
    assert lib.gdn_gemm_bf16_ws(P, 64, P, 64, P, 64, 0, None, 0, 10, 64, 64, P + 16, 1 << 20, None) == 6
    assert lib.gdn_gemm_bf16_ws(P, 64, P, 64, P, 64, 0, None, 0, 0, 64, 64, P, 1 << 20, None) == 0


def test_gemm_workspace_bytes():
    """The split tail's workspace: none for K not a multiple of 64, for empty
    shapes or when blocks of at least 4 stages would not outnumber the tail
    tiles; else two 256 x 256 fp32 slots per block, at most one block per
    compute unit (128 MiB at 256)."""
    lib = gdn.lib()
    slot = 256 * 256 * 4
    assert lib.gdn_gemm_bf16_workspace_bytes(300, 200, 5000) == 0      # K % 64
    assert lib.gdn_gemm_bf16_workspace_bytes(0, 200, 5120) == 0
    assert lib.gdn_gemm_bf16_workspace_bytes(300, 200, 192) == 0       # 2 tiles x 3 stages: no 3 blocks of 4
    for M, N, K in ((300, 200, 5120), (16640, 5120, 6144), (4300, 4000, 1024), (256, 16480, 5120)):
        n = lib.gdn_gemm_bf16_workspace_bytes(M, N, K)
        assert n % (2 * slot) == 0 and 4 * slot <= n <= 512 * slot, (M, N, K, n)


def fused_call(d, **kw):
    args = dict(x=FAKE, xld=10240, z=FAKE, zld=6144, a=FAKE, b=FAKE, gld=48, act=1, w=FAKE,
                g=FAKE, wdt=1, pool=FAKE, state=FAKE, sdt=0, slots=FAKE, hi=None, R=4, nslots=8,
                l2=1e-6, ne=1e-6, y=FAKE, ydt=1, o=None)
    args.update(kw)
    return gdn.lib().gdn_decode_fused(
        None if d is None else ctypes.byref(d), args["x"], args["xld"], args["z"], args["zld"],
        args["a"], args["b"], args["gld"], args["act"], args["w"], args["g"], args["wdt"],
        args["pool"], args["state"], args["sdt"], args["slots"], args["hi"], args["R"],
        args["nslots"], args["l2"], args["ne"], args["y"], args["ydt"], args["o"], None)


def test_decode_fused_rejects_bad_args():
    assert fused_call(None) == 1
    assert fused_call(dims(16, 48, 128, 64, 4)) == 2          # d_k != d_v
    assert fused_call(dims(1, 64, 128, 128, 4)) == 2          # 64 value heads per key head: LDS
    assert fused_call(FULL, act=2) == 3
    assert fused_call(FULL, ydt=7) == 3
    assert fused_call(FULL, sdt=2) == 3                       # state dtype
    assert fused_call(FULL, sdt=1, R=0, x=None) == 0          # bf16 state accepted
    assert fused_call(FULL, R=9) == 4                         # more requests than slots
    assert fused_call(FULL, xld=10000) == 4                   # x_ld < Cqkv
    assert fused_call(FULL, zld=6000) == 4
    assert fused_call(FULL, gld=40) == 4
    assert fused_call(FULL, l2=-1.0) == 4
    assert fused_call(FULL, x=None) == 1
    assert fused_call(FULL, y=None) == 1
    assert fused_call(FULL, state=FAKE + 4) == 6              # state not 16-byte aligned
    assert fused_call(FULL, z=FAKE + 1) == 6
    assert fused_call(FULL, R=0, x=None) == 0                 # nothing to do


def prefill_fused_call(d, **kw):
    args = dict(x=FAKE, xld=10240, z=FAKE, zld=6144, a=FAKE, b=FAKE, gld=48, act=1, w=FAKE,
                g=FAKE, wdt=1, pool=FAKE, state=FAKE, sdt=0, qsl=FAKE, slots=FAKE, hi=None, R=2, T=100,
                nslots=8, snaps=None, nsnap=0, sint=0, l2=1e-6, ne=1e-6, y=FAKE, ydt=1, ws=FAKE,
                wsb=1 << 40)
    args.update(kw)
    return gdn.lib().gdn_prefill_fused(
        None if d is None else ctypes.byref(d), args["x"], args["xld"], args["z"], args["zld"],
        args["a"], args["b"], args["gld"], args["act"], args["w"], args["g"], args["wdt"],
        args["pool"], args["state"], args["sdt"], args["qsl"], args["slots"], args["hi"], args["R"],
        args["T"], args["nslots"], args["snaps"], args["nsnap"], args["sint"], args["l2"], args["ne"],
        args["y"], args["ydt"], args["ws"], args["wsb"], None)


def test_prefill_fused_rejects_bad_args():
    need = gdn.lib().gdn_prefill_fused_workspace_bytes(ctypes.byref(FULL), 100, 2)
    assert need > 0
    assert prefill_fused_call(None) == 1
    assert prefill_fused_call(dims(16, 48, 96, 96, 4)) == 2
    assert prefill_fused_call(FULL, act=5) == 3
    assert prefill_fused_call(FULL, R=0) == 4              # tokens but no requests
    assert prefill_fused_call(FULL, xld=100) == 4
    assert prefill_fused_call(FULL, ne=-1.0) == 4
    assert prefill_fused_call(FULL, y=None) == 1
    assert prefill_fused_call(FULL, wsb=need - 1) == 5     # workspace too small
    assert prefill_fused_call(FULL, ws=None) == 5
    assert prefill_fused_call(FULL, ws=FAKE + 16) == 6     # workspace not 256-byte aligned
    assert prefill_fused_call(FULL, xld=10241) == 6        # odd row stride
    assert prefill_fused_call(FULL, T=0, R=0, x=None) == 0
    assert prefill_fused_call(FULL, sdt=4) == 3
    assert prefill_fused_call(FULL, nsnap=2, sint=48, snaps=FAKE) == 4   # not a multiple of 32
    assert prefill_fused_call(FULL, nsnap=2, sint=0, snaps=FAKE) == 4
    assert prefill_fused_call(FULL, nsnap=-1) == 4
    assert prefill_fused_call(FULL, nsnap=2, sint=64, snaps=None) == 1
    assert prefill_fused_call(FULL, nsnap=2, sint=64, snaps=FAKE + 2) == 6
    assert prefill_fused_call(FULL, sdt=1, x=FAKE + 2) == 6   # bf16 state needs 16-byte conv rows


def test_workspace_query():
    assert gdn.gdn_prefill_workspace_bytes((16, 48, 128, 128, 3), 100, 2) == 0
    n = gdn.gdn_prefill_workspace_bytes(FULL, 70000, 16)
    assert n >= 0


def test_validate_metadata_host():
    ok = gdn.gdn_validate_metadata(torch.tensor([0, 3, 3, 7]), torch.tensor([5, 0, 2]), 7, 6)
    assert ok == 0
    assert gdn.gdn_validate_metadata(torch.tensor([1, 3, 7]), torch.tensor([0, 1]), 7, 6) == 8
    assert gdn.gdn_validate_metadata(torch.tensor([0, 4, 3]), torch.tensor([0, 1]), 3, 6) == 8
    assert gdn.gdn_validate_metadata(torch.tensor([0, 3, 7]), torch.tensor([0, 0]), 7, 6) == 8
    assert gdn.gdn_validate_metadata(torch.tensor([0, 3, 7]), torch.tensor([0, 6]), 7, 6) == 8
    assert gdn.gdn_validate_metadata(torch.tensor([0, 3, 6]), torch.tensor([0, 1]), 7, 6) == 8
    assert gdn.gdn_validate_metadata(torch.tensor([0]), torch.tensor([], dtype=torch.int32), 0, 0) == 0
    rng = np.random.default_rng(0)
    perm = torch.from_numpy(rng.permutation(100000)[:50].astype(np.int32))
    qsl = torch.arange(51, dtype=torch.int32)
    assert gdn.gdn_validate_metadata(qsl, perm, 50, 100000) == 0
    perm[7] = perm[3]
    assert gdn.gdn_validate_metadata(qsl, perm, 50, 100000) == 8


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        gdn.gdn_rmsnorm(torch.zeros(4, 8), torch.ones(8), x.new_zeros(4, 8))


def spec_call(d, **kw):
    args = dict(x=FAKE, xld=10240, z=FAKE, zld=6144, a=FAKE, b=FAKE, gld=48, act=1, w=FAKE,
                g=FAKE, wdt=1, pool=FAKE, state=FAKE, sdt=0, qsl=FAKE, slots=FAKE, spec=FAKE, maxn=4,
                hi=None, R=4, T=16, nslots=32, l2=1e-6, ne=1e-6, y=FAKE, ydt=1, o=None)
    args.update(kw)
    return gdn.lib().gdn_spec_verify(
        None if d is None else ctypes.byref(d), args["x"], args["xld"], args["z"], args["zld"],
        args["a"], args["b"], args["gld"], args["act"], args["w"], args["g"], args["wdt"],
        args["pool"], args["state"], args["sdt"], args["qsl"], args["slots"], args["spec"],
        args["maxn"], args["hi"], args["R"], args["T"], args["nslots"], args["l2"], args["ne"],
        args["y"], args["ydt"], args["o"], None)


def test_spec_verify_rejects_bad_args():
    assert spec_call(None) == 1
    assert spec_call(dims(16, 48, 128, 128, 3)) == 2
    assert spec_call(FULL, maxn=0) == 4
    assert spec_call(FULL, maxn=9) == 4
    assert spec_call(FULL, T=17) == 4             # more tokens than R x max_tokens
    assert spec_call(FULL, R=33) == 4             # more requests than slots
    assert spec_call(FULL, xld=10239) == 4
    assert spec_call(FULL, gld=47) == 4
    assert spec_call(FULL, l2=-1.0) == 4
    assert spec_call(FULL, act=5) == 3
    assert spec_call(FULL, sdt=3) == 3
    assert spec_call(FULL, spec=None) == 1
    assert spec_call(FULL, y=None) == 1
    assert spec_call(FULL, state=FAKE + 4) == 6
    assert spec_call(FULL, spec=FAKE + 2) == 6
    assert spec_call(FULL, maxn=8, x=None) == 1   # 8 tokens of LDS still fit at full shapes


def test_validate_spec_metadata_host():
    def v(qsl, slots, spec, T, nslots):
        return gdn.gdn_validate_spec_metadata(torch.tensor(qsl), torch.tensor(slots),
                                              torch.tensor(spec), T, nslots)
    qsl, slots = [0, 3, 4, 6], [0, 1, 2]
    spec = [[10, 11, 12], [0 + 13, -1, -1], [14, 15, -1]]  # entries past a request's length unread
    assert v(qsl, slots, spec, 6, 16) == 0
    spec_in_place = [[0, 11, 12], [1, -1, -1], [2, 15, -1]]
    assert v(qsl, slots, spec_in_place, 6, 16) == 0
    assert v(qsl, slots, [[10, 11, 12], [11, -1, -1], [14, 15, -1]], 6, 16) == 8  # repeated
    assert v(qsl, slots, [[10, 1, 12], [13, -1, -1], [14, 15, -1]], 6, 16) == 8   # other input slot
    assert v(qsl, slots, [[10, 11, 1], [13, -1, -1], [14, 15, -1]], 6, 16) == 8
    assert v(qsl, slots, [[10, 11, 16], [13, -1, -1], [14, 15, -1]], 6, 16) == 8  # out of range
    assert v([0, 4, 4, 6], slots, [[10, 11, 12], [13, -1, -1], [14, 15, -1]], 6, 16) == 8  # too long
    assert v(qsl, [0, 1, 1], spec, 6, 16) == 8                                    # input slots repeat


def test_validate_snapshot_metadata_host():
    def v(qsl, slots, snaps, interval, T, nslots):
        return gdn.gdn_validate_snapshot_metadata(torch.tensor(qsl), torch.tensor(slots),
                                                  torch.tensor(snaps), interval, T, nslots)
    qsl, slots = [0, 70, 100, 200], [0, 1, 2]
    snaps = [[5, 6, -1], [-1, -1, -1], [7, 8, 9]]   # 70 -> 2 snapshots, 30 -> 0, 100 -> 3
    assert v(qsl, slots, snaps, 32, 200, 16) == 0
    assert v(qsl, slots, [[5, 5, -1], [-1, -1, -1], [7, 8, 9]], 32, 200, 16) == 8   # repeated
    assert v(qsl, slots, [[5, 6, -1], [-1, -1, -1], [7, 8, 2]], 32, 200, 16) == 8   # a request's slot
    assert v(qsl, slots, [[5, 16, -1], [-1, -1, -1], [7, 8, 9]], 32, 200, 16) == 8  # out of range
    assert v(qsl, slots, snaps, 48, 200, 16) == 4                                   # interval
    assert v(qsl, slots, [[5, 6, 6], [-1, -1, -1], [7, 8, 9]], 32, 200, 16) == 0    # unread entry


GQA = gdn.GqaDimsC(24, 4, 256, 64)


def gqa_call(d=GQA, **kw):
    args = dict(q=FAKE, qld=24 * 256, gate=FAKE, gld=24 * 256, k=FAKE, v=FAKE, kvld=4 * 256, act=1,
                kc=FAKE, vc=FAKE, cdt=1, ks=1.0, vs=1.0, bt=FAKE, maxp=40, lens=FAKE, R=8, npages=400, P=64,
                maxctx=2048, theta=1e4, y=FAKE, ydt=1, o=None, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    return gdn.lib().gqa_decode_paged(
        None if d is None else ctypes.byref(d), args["q"], args["qld"], args["gate"], args["gld"],
        args["k"], args["v"], args["kvld"], args["act"], args["kc"], args["vc"], args["cdt"],
        args["ks"], args["vs"], args["bt"], args["maxp"], args["lens"], args["R"], args["npages"], args["P"],
        args["maxctx"], args["theta"], args["y"], args["ydt"], args["o"], args["ws"], args["wsb"],
        None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=None), 1),
    (dict(d=gdn.GqaDimsC(24, 5, 256, 64)), 2),     # Hq % Hkv
    (dict(d=gdn.GqaDimsC(24, 2, 256, 64)), 2),     # 12 query heads per kv head
    (dict(d=gdn.GqaDimsC(24, 4, 128, 64)), 2),     # head dim
    (dict(d=gdn.GqaDimsC(24, 4, 256, 63)), 2),     # odd rotary dim
    (dict(d=gdn.GqaDimsC(24, 4, 256, 258)), 2),    # rotary dim > head dim
    (dict(act=2), 3), (dict(cdt=0), 3), (dict(cdt=3), 3), (dict(ydt=5), 3), (dict(ydt=2), 3),
    (dict(cdt=2, ks=0.0), 4), (dict(cdt=2, vs=float("inf")), 4), (dict(cdt=2, ks=float("nan")), 4),
    (dict(cdt=2, kc=FAKE + 8), 6),
    (dict(R=-1), 4), (dict(P=0), 4), (dict(maxctx=0), 4), (dict(maxp=0), 4),
    (dict(qld=24 * 256 - 1), 4), (dict(kvld=100), 4), (dict(theta=0.0), 4),
    (dict(npages=1 << 20, P=1024), 4),             # cache rows beyond 2^31
    (dict(k=None), 1), (dict(bt=None), 1), (dict(ws=None), 1),
    (dict(kc=FAKE + 8), 6), (dict(ws=FAKE + 4), 6),
    (dict(wsb=16), 5),
])
def test_gqa_decode_rejects_bad_args(kw, status):
    d = kw.pop("d", GQA)
    assert gqa_call(d, **kw) == status


def test_gqa_empty_batch_and_workspace_query():
    assert gqa_call(R=0, q=None, k=None, ws=None) == 0     # nothing to do: no pointer needed
    lib = gdn.lib()
    ws = lib.gqa_decode_workspace_bytes(ctypes.byref(GQA), 64, 3584)
    nsplit = (3584 + 511) // 512      # GQA_SPLIT_KEYS positions per partial
    # partial (max, sum) per (request, query head, run), 256-byte aligned, then the partial o
    assert ws == (64 * 24 * nsplit * 8 + 255) // 256 * 256 + 64 * 24 * nsplit * 256 * 4
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(gdn.GqaDimsC(24, 4, 128, 64)), 64, 10) == 0
    assert lib.gqa_decode_workspace_bytes(ctypes.byref(GQA), 64, 0) == 0


def test_gqa_validate_metadata_host():
    from hybrid_linear_attention_amd import gqa
    bt = np.array([[3, 0, -1], [1, 2, -1]], np.int32)
    assert gqa.gqa_validate_decode_metadata(bt, [5, 8], 5, 4, 12) == 0
    assert gqa.gqa_validate_decode_metadata(bt, [0, 8], 5, 4, 12) == 8           # empty context
    assert gqa.gqa_validate_decode_metadata(bt, [5, 9], 5, 4, 12) == 8           # past the table
    assert gqa.gqa_validate_decode_metadata(bt, [5, 8], 5, 4, 7) == 8            # past max_context_len
    assert gqa.gqa_validate_decode_metadata(bt, [5, 8], 3, 4, 12) == 8           # page id 3 >= 3
    shared = np.array([[3, 0, -1], [3, 2, -1]], np.int32)
    assert gqa.gqa_validate_decode_metadata(shared, [5, 8], 5, 4, 12) == 0       # shared read-only prefix page
    assert gqa.gqa_validate_decode_metadata(shared, [3, 8], 5, 4, 12) == 8       # request 0 appends into it


def test_prefill_fused_noalloc_rejects_on_the_host():
    """The no-allocation prefill validates like gdn_prefill_fused and refuses a
    batch beyond its static scratch (GDN_ERR_SCRATCH) before any HIP call."""
    lib = gdn.lib()

    def call(d, T, R, **kw):
        args = dict(x=FAKE, y=FAKE, act=1)
        args.update(kw)
        return lib.gdn_prefill_fused_noalloc(
            None if d is None else ctypes.byref(d), args["x"], 10240, FAKE, 6144, FAKE, FAKE, 48,
            args["act"], FAKE, FAKE, 1, FAKE, FAKE, 0, FAKE, FAKE, None, R, T, 64, None, 0, 0,
            1e-6, 1e-6, args["y"], 1, None)
    assert gdn.gdn_prefill_fused_workspace_bytes(FULL, 4096, 1) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    assert gdn.gdn_prefill_fused_workspace_bytes(FULL, 2000, 40) <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    assert call(FULL, 4096, 1) == 9                  # GDN_ERR_SCRATCH
    assert call(None, 100, 2) == 1
    assert call(dims(16, 48, 96, 96, 4), 100, 2) == 2
    assert call(FULL, 100, 2, act=5) == 3
    assert call(FULL, 100, 0) == 4
    assert call(FULL, 100, 2, y=None) == 1
    assert call(FULL, 100, 2, x=FAKE + 2) == 6       # misaligned conv rows
    assert call(FULL, 0, 0, x=None) == 0             # empty batch: nothing to do
    assert gdn.lib().gdn_status_string(9).startswith(b"GDN_ERR_SCRATCH")
