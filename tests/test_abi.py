"""libdblock's C ABI on the host: it loads, exports every declared symbol, and
rejects bad arguments with the documented status codes before touching the GPU.

No compute call is made here (no GPU is needed): every call below fails
validation, which the library performs before any HIP runtime call.
"""
import ctypes
import os

import pytest

from block_wise_decoding_amd import dblock

DEV = 1 << 40          # a fake, 256-byte-aligned "device" address: never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dblock.LIB_PATH):
        from block_wise_decoding_amd.build import build
        build()
    return dblock.load_library()


def test_exports_every_header_symbol(lib):
    names = dblock.header_symbols()
    assert set(names) == {"dblk_status_string", "dblk_abi_version", "dblk_attend_workspace_size",
                          "dblk_attend", "dblk_lmhead_workspace_size", "dblk_lmhead_confidence",
                          "dblk_threshold_commit", "dblk_threshold_commit_eos",
                          "dblk_lmhead_confidence_commit",
                          "dblk_decode_block_workspace_size", "dblk_decode_block",
                          "dblk_decode_block_run", "dblk_cache_append", "dblk_probe_read",
                          "dblk_attend_segments_workspace_size", "dblk_attend_segments",
                          "dblk_lmhead_confidence_commit_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dblk_abi_version() == 3


def test_decode_args_layout_matches_header():
    """The ctypes mirror of dblk_decode_args has the header's fields, in order."""
    import re
    txt = open(dblock.HEADER).read()
    body = re.search(r"typedef struct \{([^{}]*?)\} dblk_decode_args;", txt, re.S).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        decl = re.sub(r"^(const\s+)?(void|int32_t|float|uint8_t)\s*", "", decl)
        names += [n.strip().lstrip("*").strip() for n in decl.split(",")]
    assert names == [f[0] for f in dblock.DecodeArgs._fields_]


def test_status_strings(lib):
    for code, name in dblock.STATUS_NAMES.items():
        assert lib.dblk_status_string(code).decode().startswith(name)
    assert lib.dblk_status_string(99).decode().startswith("DBLK_ERR_?")


def test_workspace_sizes_are_pure_host(lib):
    # LLaDA-MoE-shaped block: 64 rows, d 2048, vocabulary 157184
    n = lib.dblk_lmhead_workspace_size(64, 2048, 157184)
    assert 256 < n < (1 << 22)
    assert lib.dblk_lmhead_workspace_size(0, 2048, 157184) == 0
    assert lib.dblk_lmhead_workspace_size(4096, 2048, 157184) > n
    a = lib.dblk_attend_workspace_size(1, 16, 64, 128, 768, 448)
    assert a > 0                      # few (b, h) pairs: the key range is split
    assert lib.dblk_attend_workspace_size(32, 16, 128, 128, 1024, 1536) == 0   # one split


def _attend(lib, **kw):
    a = dict(q=DEV, kp=DEV, vp=DEV, kb=DEV, vb=DEV, ks=DEV, vs=DEV, pl=None, B=1, H=2, L=64,
             D=128, P=32, S=16, S_cap=None, scale=0.0, out=DEV, ws=DEV, wsb=1 << 30, stream=None)
    a.update(kw)
    S_cap = a["S"] if a["S_cap"] is None else a["S_cap"]
    return lib.dblk_attend(a["q"], a["kp"], a["vp"], a["kb"], a["vb"], a["ks"], a["vs"], a["pl"],
                           a["B"], a["H"], a["L"], a["D"], a["P"], a["S"], S_cap, a["scale"],
                           a["out"], a["ws"], a["wsb"], a["stream"])


def test_attend_validation(lib):
    assert _attend(lib, D=96) == 2 and _attend(lib, L=40) == 2 and _attend(lib, L=256) == 2
    assert _attend(lib, B=-1) == 2 and _attend(lib, H=0) == 2 and _attend(lib, S=-3) == 2
    assert _attend(lib, P=60000, S=6000) == 2
    assert _attend(lib, scale=-1.0) == 2 and _attend(lib, scale=float("nan")) == 2
    assert _attend(lib, q=None) == 1 and _attend(lib, kb=None) == 1 and _attend(lib, out=None) == 1
    assert _attend(lib, kp=None) == 1 and _attend(lib, vs=None) == 1
    assert _attend(lib, q=DEV + 8) == 3 and _attend(lib, vb=DEV + 2) == 3
    # few (b, h) pairs: the key range is split and needs a workspace
    assert _attend(lib, P=4500, ws=None) == 4 and _attend(lib, P=4500, wsb=16) == 4
    assert _attend(lib, P=4500, ws=DEV + 16) == 3
    assert _attend(lib, B=0, q=None) == 0          # empty batch: valid no-op
    # with P = 0 and S = 0 the segment pointers may be NULL: the NULL check
    # passes and the (deliberately misaligned) query is what gets reported
    assert _attend(lib, kp=None, vp=None, ks=None, vs=None, P=0, S=0, q=DEV + 2) == 3
    assert _attend(lib, kp=None, vp=None, P=0, q=DEV + 2) == 3
    assert _attend(lib, kp=None, vp=None, P=5, q=DEV + 2) == 1
    assert _attend(lib, S=16, S_cap=8) == 2            # suffix window longer than its buffer
    assert _attend(lib, S=8, S_cap=16, q=DEV + 2) == 3  # a window is fine: misaligned q reported


def _lm(lib, **kw):
    a = dict(h=DEV, W=DEV, M=64, d=2048, V=157184, conf=DEV, amax=DEV, ws=DEV, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dblk_lmhead_confidence(a["h"], a["W"], a["M"], a["d"], a["V"], a["conf"], a["amax"],
                                      a["ws"], a["wsb"], a["stream"])


def test_lmhead_validation(lib):
    # the vocabulary is capped at 2^30 rows; nothing launches
    assert _lm(lib, d=64, V=(1 << 30) + 1) == 2
    assert _lm(lib, M=128, d=64, V=1 << 30, wsb=100) == 4
    assert _lm(lib, d=100) == 2 and _lm(lib, d=32) == 2 and _lm(lib, V=0) == 2 and _lm(lib, M=-1) == 2
    assert _lm(lib, d=32768) == 2
    # the many-row path addresses h by 32-bit byte offsets: h past 2 GiB is refused
    assert _lm(lib, M=1 << 17, d=16384, wsb=1 << 40) == 2
    assert _lm(lib, h=None) == 1 and _lm(lib, W=None) == 1 and _lm(lib, conf=None) == 1
    assert _lm(lib, h=DEV + 2) == 3 and _lm(lib, conf=DEV + 1) == 3
    assert _lm(lib, ws=None) == 4 and _lm(lib, wsb=100) == 4 and _lm(lib, ws=DEV + 64) == 3
    assert _lm(lib, M=0, h=None) == 0


def _commit(lib, **kw):
    a = dict(conf=DEV, amax=DEV, tok=DEV, mask=DEV, B=2, L=64, tau=0.9, n=None, stream=None)
    a.update(kw)
    return lib.dblk_threshold_commit(a["conf"], a["amax"], a["tok"], a["mask"], a["B"], a["L"],
                                     a["tau"], a["n"], a["stream"])


def test_commit_validation(lib):
    assert _commit(lib, L=0) == 2 and _commit(lib, L=5000) == 2 and _commit(lib, B=-2) == 2
    assert _commit(lib, conf=None) == 1 and _commit(lib, mask=None) == 1
    assert _commit(lib, tok=DEV + 2) == 3 and _commit(lib, n=DEV + 1) == 3
    assert _commit(lib, B=0, conf=None) == 0


def _lmc(lib, **kw):
    a = dict(h=DEV, W=DEV, d=2048, V=157184, conf=DEV, amax=DEV, tok=DEV, mask=DEV, B=1, L=64,
             tau=0.9, n=None, ws=DEV, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dblk_lmhead_confidence_commit(a["h"], a["W"], a["d"], a["V"], a["conf"], a["amax"],
                                             a["tok"], a["mask"], a["B"], a["L"], a["tau"], a["n"],
                                             a["ws"], a["wsb"], a["stream"])


def test_lmhead_commit_validation(lib):
    assert _lmc(lib, d=100) == 2 and _lmc(lib, L=0) == 2 and _lmc(lib, L=5000) == 2
    assert _lmc(lib, V=0) == 2 and _lmc(lib, B=-1) == 2
    assert _lmc(lib, h=None) == 1 and _lmc(lib, tok=None) == 1 and _lmc(lib, mask=None) == 1
    assert _lmc(lib, h=DEV + 2) == 3 and _lmc(lib, tok=DEV + 2) == 3 and _lmc(lib, n=DEV + 1) == 3
    assert _lmc(lib, ws=None) == 4 and _lmc(lib, wsb=64) == 4 and _lmc(lib, ws=DEV + 16) == 3
    assert _lmc(lib, B=0, h=None) == 0


def _eos(lib, **kw):
    a = dict(conf=DEV, amax=DEV, tok=DEV, mask=DEV, B=2, L=64, tau=0.9, eos=7, n=None, fin=None,
             stream=None)
    a.update(kw)
    return lib.dblk_threshold_commit_eos(a["conf"], a["amax"], a["tok"], a["mask"], a["B"], a["L"],
                                         a["tau"], a["eos"], a["n"], a["fin"], a["stream"])


def test_commit_eos_validation(lib):
    assert _eos(lib, L=0) == 2 and _eos(lib, eos=-1) == 2 and _eos(lib, B=-1) == 2
    assert _eos(lib, conf=None) == 1 and _eos(lib, tok=DEV + 2) == 3
    assert _eos(lib, B=0, conf=None) == 0


def _decode_args(**kw):
    a = dict(q=DEV, k_prefix=DEV, v_prefix=DEV, k_block=DEV, v_block=DEV, k_suffix=DEV,
             v_suffix=DEV, prefix_len=None, B=1, H=16, L=64, D=128, P_cap=768, S=448, S_cap=448,
             scale=0.0, attn_out=DEV, h=DEV, W=DEV, d=2048, V=157184, conf=DEV, argmax=DEV,
             tokens=DEV, mask=DEV, threshold=0.9, eos_id=-1, max_iters=0, commit_iter=None,
             n_iters=None, finished=None)
    a.update(kw)
    return dblock.DecodeArgs(**a)


def test_decode_block_validation(lib):
    ws_n = lib.dblk_decode_block_workspace_size(ctypes.byref(_decode_args()))
    lm_n = lib.dblk_lmhead_workspace_size(64, 2048, 157184)
    at_n = lib.dblk_attend_workspace_size(1, 16, 64, 128, 768, 448)
    assert ws_n >= lm_n + at_n + 4 and ws_n % 256 == 0
    assert lib.dblk_decode_block_workspace_size(None) == 0

    def run(wsb=1 << 30, ws=DEV, **kw):
        return lib.dblk_decode_block(ctypes.byref(_decode_args(**kw)), ws, wsb, None)

    assert lib.dblk_decode_block(None, DEV, 1 << 30, None) == 1
    assert run(D=96) == 2 and run(L=40) == 2 and run(S=500) == 2 and run(d=100) == 2
    assert run(q=None) == 1 and run(h=None) == 1 and run(tokens=None) == 1 and run(mask=None) == 1
    assert run(q=DEV + 2) == 3 and run(W=DEV + 8) == 3 and run(commit_iter=DEV + 2) == 3
    assert run(ws=None) == 4 and run(wsb=ws_n - 1) == 4 and run(ws=DEV + 64) == 3
    assert run(scale=-1.0) == 2
    assert run(B=0, q=None) == 0

    host = (ctypes.c_int32 * 2)()
    n = ctypes.c_int32(-1)

    def run_p(chunk=4, flags=ctypes.addressof(host), wsb=1 << 30, ws=DEV, **kw):
        return lib.dblk_decode_block_run(ctypes.byref(_decode_args(**kw)), chunk, flags, ws, wsb,
                                         None, ctypes.byref(n))

    assert run_p(chunk=0) == 2 and run_p(D=96) == 2 and run_p(q=None) == 1
    assert run_p(flags=None) == 1 and run_p(flags=ctypes.addressof(host) + 2) == 3
    assert run_p(wsb=16) == 4 and run_p(ws=DEV + 8) == 3
    assert run_p(B=0, q=None) == 0 and n.value == 0


def _append(lib, **kw):
    a = dict(kp=DEV, vp=DEV, kb=DEV, vb=DEV, pl=DEV, B=2, H=4, L=64, D=128, P_cap=256,
             app=None, stream=None)
    a.update(kw)
    return lib.dblk_cache_append(a["kp"], a["vp"], a["kb"], a["vb"], a["pl"], a["B"], a["H"],
                                 a["L"], a["D"], a["P_cap"], a["app"], a["stream"])


def test_cache_append_validation(lib):
    assert _append(lib, D=96) == 2 and _append(lib, L=0) == 2 and _append(lib, P_cap=32) == 2
    assert _append(lib, H=0) == 2 and _append(lib, B=70000) == 2
    assert _append(lib, kp=None) == 1 and _append(lib, pl=None) == 1
    assert _append(lib, kb=DEV + 2) == 3 and _append(lib, pl=DEV + 1) == 3
    assert _append(lib, app=DEV + 2) == 3
    assert _append(lib, B=0, kp=None) == 0


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        dblock.dblk_lmhead_confidence(x, x, torch.zeros(4), torch.zeros(4, dtype=torch.int32))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        dblock.load_library(str(tmp_path / "nope.so"))


def test_probe_read_validation(lib):
    sink = DEV
    ok = dict(buf=DEV, nbytes=1 << 20, nt=1, grid=256, sink=sink)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.dblk_probe_read(a["buf"], a["nbytes"], a["nt"], a["grid"], a["sink"], None)

    assert call(nbytes=0) == 2 and call(nbytes=(1 << 20) + 16) == 2
    assert call(grid=0) == 2 and call(grid=65536) == 2
    assert call(buf=None) == 1 and call(sink=None) == 1
    assert call(buf=DEV + 8) == 3 and call(sink=DEV + 2) == 3


def test_segment_structs_match_the_c_layout(tmp_path):
    """ctypes mirrors of dblk_kv_segment / dblk_attend_args: every field at the
    offset a C compiler gives it, and the same sizes."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    fields_seg = [f[0] for f in dblock.KVSegment._fields_]
    fields_args = [f[0] for f in dblock.AttendArgs._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "dblock.h"', "int main(void) {",
           'printf("%zu %zu\\n", sizeof(dblk_kv_segment), sizeof(dblk_attend_args));']
    src += [f'printf("%zu\\n", offsetof(dblk_kv_segment, {n}));' for n in fields_seg]
    src += [f'printf("%zu\\n", offsetof(dblk_attend_args, {n}));' for n in fields_args]
    src += ["return 0; }"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", dblock.INCLUDE, str(c), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    vals = [int(x) for x in out]
    assert vals[0] == ctypes.sizeof(dblock.KVSegment) and vals[1] == ctypes.sizeof(dblock.AttendArgs)
    want = [getattr(dblock.KVSegment, n).offset for n in fields_seg] + \
           [getattr(dblock.AttendArgs, n).offset for n in fields_args]
    assert vals[2:] == want


def _seg_args(**kw):
    B, H, L, D = kw.pop("B", 2), kw.pop("H", 2), kw.pop("L", 64), kw.pop("D", 128)

    def seg(n, k=DEV, sb=None, sh=None, st=None, lpb=None):
        st = D if st is None else st
        sh = n * D if sh is None else sh
        sb = H * n * D if sb is None else sb
        return dblock.KVSegment(k, k, sb, sh, st, n, lpb)

    pre = kw.pop("prefix", seg(32))
    blk = kw.pop("block", seg(L))
    suf = kw.pop("suffix", seg(16))
    a = dblock.AttendArgs(B, H, L, D, kw.pop("q", DEV), L * H * D, H * D, D, pre, blk, suf,
                          kw.pop("scale", 0.0), kw.pop("out", DEV), L * H * D, H * D, D)
    for k, v in kw.items():
        setattr(a, k, v)
    return a, seg


def test_attend_segments_validation(lib):
    def call(a):
        return lib.dblk_attend_segments(ctypes.byref(a), DEV, 1 << 30, None)

    a, seg = _seg_args(B=0)
    assert call(a) == 0                                   # B == 0: valid no-op
    assert lib.dblk_attend_segments(None, DEV, 1 << 30, None) == 1
    for kw, code in [(dict(D=96), 2), (dict(L=40), 2), (dict(H=0), 2), (dict(B=70000), 2),
                     (dict(scale=-1.0), 2), (dict(q=None), 1), (dict(out=None), 1),
                     (dict(q=DEV + 8), 3), (dict(q_stride_h=100), 3), (dict(o_stride_l=-8), 3)]:
        a, seg = _seg_args(**kw)
        assert call(a) == code, kw
    a, seg = _seg_args()
    for bad, code in [(seg(-1), 2), (seg(32, k=None), 1), (seg(32, k=DEV + 2), 3),
                      (seg(32, st=12), 3), (seg(32, lpb=DEV + 1), 3), (seg(70000), 2),
                      (seg(32, sb=1 << 45), 2), (seg(32, st=1 << 24), 2)]:
        a, _ = _seg_args(prefix=bad)
        assert call(a) == code, (bad.len, bad.stride_t)
    a, _ = _seg_args(prefix=seg(0, k=None), suffix=seg(0, k=None))   # empty segments need no pointer
    assert lib.dblk_attend_segments_workspace_size(ctypes.byref(a)) >= 0
    a, _ = _seg_args(prefix=seg(40000), suffix=seg(30000))            # T_cap > 65536
    assert call(a) == 2


def test_noalloc_validation(lib):
    """The allocation-free LM-head call validates like the workspace call and
    refuses, before any HIP call, a shape whose scratch would pass the
    library's fixed array."""
    def call(B=1, L=64, d=2048, V=157184, h=DEV, conf=DEV):
        return lib.dblk_lmhead_confidence_commit_noalloc(h, DEV, d, V, conf, DEV, DEV, DEV, B, L,
                                                         0.9, None, None)
    assert call(d=100) == 2 and call(L=5000) == 2
    assert call(h=None) == 1 and call(conf=DEV + 2) == 3
    assert call(B=0) == 0
    import re
    m = re.search(r"#define DBLK_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(dblock.HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == dblock.NOALLOC_SCRATCH_BYTES
    assert dblock.lmhead_workspace_size(64 * 64, 128, 157184) > dblock.NOALLOC_SCRATCH_BYTES
    assert call(B=64, L=64, d=128) == 4                 # DBLK_ERR_WORKSPACE
