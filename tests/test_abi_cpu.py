"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments before any HIP call.

Pointers here are fake but aligned host integers; the library only compares
them (null, alignment, overlap) and never dereferences or launches on a
rejected call.  No call in this file reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

from attention_shards_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")



def test_library_is_built():
    """The library must exist: a missing build fails here instead of
    leaving the rest of this file unrun."""
    assert os.path.exists(B.LIB_PATH), f"{B.LIB_PATH} is not built"


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    src = re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", src)))


def enum_values():
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"\b(TP_(?:SUCCESS|ERR_[A-Z_]+))\s*=\s*(\d+)", header_text())}


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    v = int(re.search(r"#define TP_ABI_VERSION (\d+)", header_text()).group(1))
    assert lib.tp_abi_version() == v
    vals = enum_values()
    assert len(vals) == 11
    for name, code in vals.items():
        assert lib.tp_status_string(code).decode() == name
        assert B.STATUS[code] == name
    assert lib.tp_status_string(999).decode() == "TP_ERR_UNKNOWN_STATUS"


def test_workspace_queries(lib):
    assert lib.tp_ffn_shard_workspace_bytes(4096, 4096, 16384, 8, B.TP_BF16) == 4096 * 2048 * 2
    assert lib.tp_ffn_shard_workspace_bytes(128, 1024, 4096, 1, B.TP_F32) == 128 * 4096 * 4
    # bf16: GeLU(Z_i) columns rounded up to a multiple of 64 (its K-blocked
    # layout), then a 256-byte granule: 3 x 64 x 2 = 384 -> 512
    assert lib.tp_ffn_shard_workspace_bytes(3, 8, 24, 3, B.TP_BF16) == 512
    assert lib.tp_ffn_shard_workspace_bytes(2000, 3000, 2936, 1, B.TP_BF16) == 2000 * 2944 * 2
    assert lib.tp_ffn_shard_workspace_bytes(3, 8, 24, 3, B.TP_F32) == 256    # fp32: row-major
    # bf16 shards of at least 20480 ffn columns also hold X K-blocked (hidden
    # rounded up to 64 columns): 2048 x 22528 x 2 after GeLU(Z) of 2048 x 90112
    assert lib.tp_ffn_shard_workspace_bytes(2048, 22528, 90112, 1, B.TP_BF16) == \
        2048 * 90112 * 2 + 2048 * 22528 * 2
    # ... and, when GEMM2's plan splits K (here [100 x 1000] over 20480 or
    # 20472 columns: 256x256 tiles over 8 parts of K), its fp32 partials
    split = 8 * 100 * 1000 * 4
    assert lib.tp_ffn_shard_workspace_bytes(100, 1000, 20480, 1, B.TP_BF16) == \
        (100 * 20480 * 2 + 255) // 256 * 256 + (100 * 1024 * 2 + 255) // 256 * 256 + split
    assert lib.tp_ffn_shard_workspace_bytes(100, 1000, 20472 * 2, 2, B.TP_BF16) == \
        (100 * 20480 * 2 + 255) // 256 * 256 + split             # 20472 < 20480 columns
    # the hidden-10240 t=1 sweep shard: GEMM2 [2048 x 10240] over K = 40960
    # runs one wave of 256x256 tiles over 8192 columns and the other 2048
    # columns as 256x256 tiles over 4 parts of K
    assert lib.tp_ffn_shard_workspace_bytes(2048, 10240, 40960, 1, B.TP_BF16) == \
        2048 * 40960 * 2 + 2048 * 10240 * 2 + 4 * 2048 * 2048 * 4
    # a wave of full tiles leaves nothing to split (the t=8 hidden-4096 shard,
    # the headline hidden-22528 shard above)
    assert lib.tp_ffn_shard_workspace_bytes(4096, 4096, 16384, 8, B.TP_BF16) == 4096 * 2048 * 2
    assert lib.tp_ffn_shard_workspace_bytes(10, 8, 20, 3, B.TP_BF16) == 0    # t does not divide f
    assert lib.tp_ffn_shard_workspace_bytes(10, 8, 16, 0, B.TP_BF16) == 0
    # attention: 4 x [heads, seq_pad, 128] 16-bit (Q, K, V^T hi, V^T lo) + O
    # [tokens, nl*128] as fp16 + bf8 (3 bytes per element), then fp32 partial results (qb x (128 + 2) floats) for every workgroup of
    # the larger split: at seq 2048, 8 heads, both use 256-query blocks; the
    # causal one cuts the key ranges (4, 8, ..., 32 tiles) into chunks of 5
    # tiles: 32 chunks x 8 heads = 256 workgroups (the full one: 8 query
    # blocks x 4 chunks of 8 tiles x 8 heads = 256)
    split = 256 * 256 * 130 * 4
    want = 4 * 8 * 2048 * 128 * 2 + 2048 * 1024 * 3 + split
    assert lib.tp_attn_shard_workspace_bytes(1, 2048, 64, 128, 8) == want
    ragged = lib.tp_attn_shard_workspace_bytes(2, 100, 4, 128, 2)
    # one query block, one chunk, 2 sequences x 2 heads = 4 workgroups
    assert ragged == 4 * 2 * 2 * 128 * 128 * 2 + 2 * 100 * 256 * 3 + 4 * 128 * 130 * 4
    assert lib.tp_attn_shard_workspace_bytes(1, 8, 6, 128, 4) == 0


def test_workspace_queries_reject_what_the_calls_reject(lib):
    """Shapes the entry points refuse for their size give 0, never a
    wrapped product (and the attention query never plans such a shape)."""
    big = (1 << 31) - 4
    assert lib.tp_ffn_shard_workspace_bytes(1 << 31, 64, 128, 1, B.TP_BF16) == 0
    assert lib.tp_ffn_shard_workspace_bytes(big, big, 2 * big, 2, B.TP_F32) == 0
    assert lib.tp_ffn_shard_workspace_bytes(1 << 40, 8, 1 << 40, 1 << 10, B.TP_F32) == 0
    assert lib.tp_ffn_shard_reduce_workspace_bytes(big, big, 2 * big, 2, B.TP_F32) == 0
    assert lib.tp_attn_shard_workspace_bytes(1 << 20, 1 << 12, 8, 128, 1) == 0
    assert lib.tp_attn_shard_workspace_bytes(1 << 40, 0, 8, 128, 1) == 0
    assert lib.tp_attn_shard_workspace_bytes(1, 1 << 23, 8, 128, 1) == 0
    assert lib.tp_attn_shard_workspace_bytes(1, 1 << 22, 1 << 14, 128, 1) == 0
    assert lib.tp_attn_shard_workspace_bytes(1, 2048, 8, 64, 1) == 0
    # the largest accepted sequence still has a size
    assert lib.tp_attn_shard_workspace_bytes(1, (1 << 23) - 64, 1, 128, 1) > 0


# fake, 16-byte aligned, non-overlapping device addresses
X, W1, W2, Y, WS = (0x10_0000_0000 * k for k in range(1, 6))


def ffn(lib, **kw):
    a = dict(X=X, W1=W1, W2=W2, Y=Y, tokens=64, hidden=64, ffn=256, i=0, t=2,
             ld=0, din=B.TP_BF16, dout=B.TP_BF16, ws=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    st = lib.tp_ffn_shard(a["X"], a["W1"], a["W2"], a["Y"], a["tokens"], a["hidden"],
                          a["ffn"], a["i"], a["t"], a["ld"], a["din"], a["dout"],
                          a["ws"], a["wsb"], a["stream"])
    return st, lib.tp_last_error_message().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(din=7), "TP_ERR_DTYPE"),
    (dict(dout=-1), "TP_ERR_DTYPE"),
    (dict(i=2), "TP_ERR_SHARD"),
    (dict(i=-1), "TP_ERR_SHARD"),
    (dict(t=0), "TP_ERR_SHARD"),
    (dict(tokens=-1), "TP_ERR_SHAPE"),
    (dict(hidden=0), "TP_ERR_SHAPE"),
    (dict(ffn=255), "TP_ERR_DIVISIBILITY"),
    (dict(hidden=60), "TP_ERR_SHAPE"),              # not a multiple of 8 bf16
    (dict(ffn=2 * 36), "TP_ERR_SHAPE"),             # f/t = 36
    (dict(ld=100), "TP_ERR_SHAPE"),                 # ld_w1 < f/t
    (dict(ld=132), "TP_ERR_SHAPE"),                 # ld_w1 not a multiple of 8
    (dict(hidden=1 << 22, ffn=2 << 22), "TP_ERR_SHAPE"),  # bf16 row stride limits
    (dict(ffn=2 << 22), "TP_ERR_SHAPE"),
    (dict(ld=1 << 24), "TP_ERR_SHAPE"),
    # fp32 dimensions are each below 2^31, but no operand may pass 2^60
    # elements (its byte extent would wrap int64 in the alias checks)
    (dict(din=B.TP_F32, dout=B.TP_F32, tokens=(1 << 31) - 1, hidden=(1 << 31) - 4,
          ffn=2 * 64), "TP_ERR_SHAPE"),
    (dict(din=B.TP_F32, dout=B.TP_F32, hidden=1 << 30, ld=1 << 40), "TP_ERR_SHAPE"),
    (dict(X=None), "TP_ERR_NULL"),
    (dict(Y=None), "TP_ERR_NULL"),
    (dict(ws=None), "TP_ERR_WORKSPACE"),
    (dict(wsb=64 * 128 * 2 - 1), "TP_ERR_WORKSPACE"),
    (dict(W2=W2 + 8), "TP_ERR_ALIGNMENT"),
    (dict(Y=X + 64), "TP_ERR_ALIAS"),               # output inside X
    (dict(Y=WS), "TP_ERR_ALIAS"),                   # output on the workspace
    (dict(ws=W1 + 1024), "TP_ERR_ALIAS"),           # workspace inside W1_i
])
def test_ffn_rejects(lib, kw, code):
    st, msg = ffn(lib, **kw)
    assert B.STATUS[st] == code, msg
    assert msg


def test_ffn_output_in_the_padded_workspace_tail_is_an_alias(lib):
    """bf16 GeLU(Z_i) is written K-blocked over ffn/t rounded up to 64
    columns: with ffn/t = 72 the workspace extent is tokens x 128 columns,
    so an output placed just past tokens x 72 columns still overlaps it."""
    tokens, fs = 64, 72
    need = lib.tp_ffn_shard_workspace_bytes(tokens, 64, 2 * fs, 2, B.TP_BF16)
    assert need == tokens * 128 * 2
    st, msg = ffn(lib, ffn=2 * fs, Y=WS + tokens * fs * 2)
    assert B.STATUS[st] == "TP_ERR_ALIAS", msg
    st, msg = ffn(lib, ffn=2 * fs, Y=WS + need, tokens=0)
    assert st == 0, msg


def test_ffn_error_message_names_shard(lib):
    st, msg = ffn(lib, X=None, i=1)
    assert B.STATUS[st] == "TP_ERR_NULL" and "i=1" in msg


def test_ffn_fp32_vector_rule(lib):
    # 68 % 4 == 0 passes the shape rule and stops at the (later) NULL check
    st, _ = ffn(lib, din=B.TP_F32, hidden=68, ffn=2 * 68, X=None)
    assert B.STATUS[st] == "TP_ERR_NULL"
    st, _ = ffn(lib, din=B.TP_F32, hidden=66, ffn=2 * 68)
    assert B.STATUS[st] == "TP_ERR_SHAPE"


def test_ffn_zero_tokens_is_a_no_op(lib):
    st, msg = ffn(lib, tokens=0, X=None, Y=None, ws=None)
    assert st == 0, msg


def attn(lib, **kw):
    a = dict(X=X, Wqkv=W1, Wo=W2, Y=Y, batch=1, seq=128, hidden=256, nh=4, d=128,
             i=0, t=2, causal=1, din=B.TP_BF16, dout=B.TP_F32, ws=WS, wsb=1 << 30)
    a.update(kw)
    st = lib.tp_attn_shard(a["X"], a["Wqkv"], a["Wo"], a["Y"], a["batch"], a["seq"],
                           a["hidden"], a["nh"], a["d"], a["i"], a["t"], a["causal"],
                           a["din"], a["dout"], a["ws"], a["wsb"], None)
    return st, lib.tp_last_error_message().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(din=B.TP_F32), "TP_ERR_UNSUPPORTED"),
    (dict(dout=3), "TP_ERR_DTYPE"),
    (dict(i=5), "TP_ERR_SHARD"),
    (dict(nh=6, t=4), "TP_ERR_DIVISIBILITY"),
    (dict(d=64), "TP_ERR_UNSUPPORTED"),
    (dict(hidden=250), "TP_ERR_SHAPE"),
    (dict(causal=2), "TP_ERR_SHAPE"),
    (dict(seq=-3), "TP_ERR_SHAPE"),
    (dict(seq=1 << 23), "TP_ERR_SHAPE"),            # V^T rows addressed with 32-bit offsets
    (dict(hidden=1 << 22), "TP_ERR_SHAPE"),
    (dict(batch=1 << 20, seq=1 << 12), "TP_ERR_SHAPE"),   # batch*seq = 2^32
    (dict(batch=1 << 31, seq=0), "TP_ERR_SHAPE"),
    (dict(batch=1 << 16, seq=1 << 14, nh=2048, t=1), "TP_ERR_SHAPE"),  # key tiles x heads
    (dict(Wo=None), "TP_ERR_NULL"),
    (dict(wsb=1000), "TP_ERR_WORKSPACE"),
    (dict(Y=X), "TP_ERR_ALIAS"),
    (dict(ws=X + 4096), "TP_ERR_ALIAS"),
    (dict(X=X + 2), "TP_ERR_ALIGNMENT"),
])
def test_attn_rejects(lib, kw, code):
    st, msg = attn(lib, **kw)
    assert B.STATUS[st] == code, msg


def test_attn_empty_is_a_no_op(lib):
    assert attn(lib, seq=0, X=None)[0] == 0
    assert attn(lib, batch=0, ws=None)[0] == 0


def reduce_call(lib, parts, t=None, R=None, out=Y, rows=32, cols=64, pdt=B.TP_BF16,
                rdt=B.TP_BF16, odt=B.TP_F32):
    t = len(parts) if t is None else t
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts) if parts else None
    st = lib.tp_partial_reduce(arr, t, R, out, rows, cols, pdt, rdt, odt, None)
    return st, lib.tp_last_error_message().decode()


def test_reduce_rejects(lib):
    P = [X, W1, W2]
    assert B.STATUS[reduce_call(lib, P, t=0)[0]] == "TP_ERR_SHARD"
    assert B.STATUS[reduce_call(lib, P * 22, t=65)[0]] == "TP_ERR_SHARD"
    assert B.STATUS[reduce_call(lib, P, cols=60)[0]] == "TP_ERR_SHAPE"
    assert B.STATUS[reduce_call(lib, P, rows=-1)[0]] == "TP_ERR_SHAPE"
    assert B.STATUS[reduce_call(lib, P, rows=1 << 40, cols=1 << 40)[0]] == "TP_ERR_SHAPE"
    assert B.STATUS[reduce_call(lib, P, pdt=9)[0]] == "TP_ERR_DTYPE"
    assert B.STATUS[reduce_call(lib, P, R=WS, rdt=4)[0]] == "TP_ERR_DTYPE"
    assert B.STATUS[reduce_call(lib, [X, 0, W2])[0]] == "TP_ERR_NULL"
    assert B.STATUS[reduce_call(lib, P, out=None)[0]] == "TP_ERR_NULL"
    assert B.STATUS[reduce_call(lib, [X, W1 + 4])[0]] == "TP_ERR_ALIGNMENT"
    # out overlapping a partial without being exactly it
    assert B.STATUS[reduce_call(lib, [X, W1], out=W1 + 256)[0]] == "TP_ERR_ALIAS"
    # same address but different element size (bf16 partial, fp32 out)
    assert B.STATUS[reduce_call(lib, [X, W1], out=W1)[0]] == "TP_ERR_ALIAS"
    assert B.STATUS[reduce_call(lib, [X], R=WS, out=WS + 16)[0]] == "TP_ERR_ALIAS"


def reduce_slice_call(lib, parts, slice_, nslices, R=None, out=Y, rows=32, cols=64,
                      pdt=B.TP_BF16, rdt=B.TP_BF16, odt=B.TP_F32):
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts) if parts else None
    st = lib.tp_partial_reduce_slice(arr, len(parts), R, out, rows, cols, slice_, nslices,
                                     pdt, rdt, odt, None)
    return st, lib.tp_last_error_message().decode()


def test_reduce_slice_rejects(lib):
    P = [X, W1, W2]
    for s, n in [(-1, 4), (4, 4), (0, 0)]:
        st, msg = reduce_slice_call(lib, P, s, n)
        assert B.STATUS[st] == "TP_ERR_SHARD" and "tp_partial_reduce_slice" in msg
    assert B.STATUS[reduce_slice_call(lib, P, 0, 2, cols=60)[0]] == "TP_ERR_SHAPE"
    assert B.STATUS[reduce_slice_call(lib, P, 0, 2, pdt=5)[0]] == "TP_ERR_DTYPE"
    assert B.STATUS[reduce_slice_call(lib, [X, 0], 1, 2)[0]] == "TP_ERR_NULL"
    # slice 1 of 2 covers rows 16..31: partials[1]'s block is W1 + [2048, 4096)
    # bytes; a bf16 out at W1 + 1024 has its block at W1 + [3072, 5120)
    assert B.STATUS[reduce_slice_call(lib, [X, W1], 1, 2, out=W1 + 1024,
                                      odt=B.TP_BF16)[0]] == "TP_ERR_ALIAS"


def test_reduce_slice_empty_block_is_a_no_op(lib):
    # rows = 2 split 4 ways: slices 2 and 3 are empty and touch nothing
    assert reduce_slice_call(lib, [None], 3, 4, out=None, rows=2)[0] == 0


def test_reduce_empty_is_a_no_op(lib):
    assert reduce_call(lib, [X, W1], rows=0)[0] == 0
    assert reduce_call(lib, [X, W1], cols=0, out=None)[0] == 0


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libtpshard.so")
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.load()


P1, P3, RR = (0x10_0000_0000 * k for k in range(7, 10))   # more fake addresses


def ffn_reduce(lib, **kw):
    a = dict(X=X, W1=W1, W2=W2, peers=[None, P1, 0x10_0000_0000 * 12, P3], R=RR, out=Y,
             tokens=64, hidden=64, ffn=256, i=0, t=4, ld=0, din=B.TP_BF16,
             pdt=B.TP_BF16, rdt=B.TP_BF16, odt=B.TP_F32, ws=WS, wsb=1 << 30)
    a.update(kw)
    peers = a["peers"]
    arr = (ctypes.c_void_p * len(peers))(*peers) if peers is not None else None
    st = lib.tp_ffn_shard_reduce(a["X"], a["W1"], a["W2"], arr, a["R"], a["out"],
                                 a["tokens"], a["hidden"], a["ffn"], a["i"], a["t"], a["ld"],
                                 a["din"], a["pdt"], a["rdt"], a["odt"], a["ws"], a["wsb"],
                                 None)
    return st, lib.tp_last_error_message().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(pdt=5), "TP_ERR_DTYPE"),
    (dict(rdt=5), "TP_ERR_DTYPE"),
    (dict(odt=5), "TP_ERR_DTYPE"),
    (dict(t=65, ffn=65 * 8, peers=[P1] * 65), "TP_ERR_SHARD"),
    (dict(i=4), "TP_ERR_SHARD"),
    (dict(ffn=250), "TP_ERR_DIVISIBILITY"),
    (dict(hidden=60), "TP_ERR_SHAPE"),
    (dict(X=None), "TP_ERR_NULL"),
    (dict(peers=None), "TP_ERR_NULL"),
    (dict(peers=[None, P1, None, P3]), "TP_ERR_NULL"),     # a peer other than i missing
    (dict(ws=None), "TP_ERR_WORKSPACE"),
    (dict(peers=[None, P1 + 4, P1 + (1 << 20), P3]), "TP_ERR_ALIGNMENT"),
    (dict(R=RR + 8), "TP_ERR_ALIGNMENT"),
    (dict(out=X + 64), "TP_ERR_ALIAS"),                    # output inside X
    (dict(out=P1 + 256), "TP_ERR_ALIAS"),                  # output inside a peer
    (dict(out=P1), "TP_ERR_ALIAS"),                        # same address, fp32 over bf16
    (dict(out=RR + 16), "TP_ERR_ALIAS"),                   # output inside the residual
    (dict(ws=P3 + 1024), "TP_ERR_ALIAS"),                  # workspace inside a peer
    (dict(ws=RR), "TP_ERR_ALIAS"),                         # workspace on the residual
    (dict(out=WS + 64 * 64 * 2 + 512), "TP_ERR_ALIAS"),    # output on the fp32 sum area
])
def test_ffn_reduce_rejects(lib, kw, code):
    st, msg = ffn_reduce(lib, **kw)
    assert B.STATUS[st] == code, msg
    assert msg


def test_ffn_reduce_workspace_query(lib):
    z = 4096 * 2048 * 2
    assert lib.tp_ffn_shard_reduce_workspace_bytes(4096, 4096, 16384, 8, B.TP_BF16) == \
        z + 4096 * 4096 * 4
    assert lib.tp_ffn_shard_reduce_workspace_bytes(10, 8, 20, 3, B.TP_BF16) == 0


def test_ffn_reduce_small_workspace(lib):
    need = lib.tp_ffn_shard_reduce_workspace_bytes(64, 64, 256, 4, B.TP_BF16)
    st, msg = ffn_reduce(lib, wsb=need - 1)
    assert B.STATUS[st] == "TP_ERR_WORKSPACE", msg


def test_ffn_reduce_zero_tokens_is_a_no_op(lib):
    st, msg = ffn_reduce(lib, tokens=0, X=None, out=None, ws=None, peers=None)
    assert st == 0, msg


def noalloc(lib, **kw):
    a = dict(X=X, W1=W1, W2=W2, Y=Y, tokens=64, hidden=64, ffn=256, i=0, t=2,
             ld=0, din=B.TP_BF16, dout=B.TP_BF16)
    a.update(kw)
    st = lib.tp_ffn_shard_noalloc(a["X"], a["W1"], a["W2"], a["Y"], a["tokens"], a["hidden"],
                                  a["ffn"], a["i"], a["t"], a["ld"], a["din"], a["dout"], None)
    return st, lib.tp_last_error_message().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(din=7), "TP_ERR_DTYPE"),
    (dict(i=2), "TP_ERR_SHARD"),
    (dict(ffn=255), "TP_ERR_DIVISIBILITY"),
    (dict(hidden=60), "TP_ERR_SHAPE"),
    (dict(X=None), "TP_ERR_NULL"),
    (dict(W2=W2 + 8), "TP_ERR_ALIGNMENT"),
    (dict(Y=X + 64), "TP_ERR_ALIAS"),
    # GeLU(Z_i) of 8192 x 8192 bf16 = 128 MiB, above the 64 MiB array
    (dict(tokens=8192, ffn=8192, t=1), "TP_ERR_WORKSPACE"),
])
def test_ffn_noalloc_rejects_before_any_hip_call(lib, kw, code):
    st, msg = noalloc(lib, **kw)
    assert B.STATUS[st] == code, msg
    assert msg


def test_ffn_noalloc_limit_matches_header(lib):
    m = re.search(r"#define TP_FFN_NOALLOC_MAX_WORKSPACE \(\(size_t\)(\d+) << (\d+)\)",
                  header_text())
    assert int(m.group(1)) << int(m.group(2)) == B.TP_FFN_NOALLOC_MAX_WORKSPACE
    # 2048 tokens x 16384 bf16 columns of GeLU(Z) fill the 64 MiB exactly
    # (hidden 8192: GEMM2 is one wave of 256x256 tiles, no split K);
    # 2048 x 16448 do not fit, nor do 1024 x 22528 (44 MiB of GeLU(Z) plus
    # the K-blocked copy of 1024 x 16384 X, 32 MiB), nor 2048 x 16384 with
    # hidden 64 (GEMM2 then splits K: 4 MiB of partials on top)
    assert lib.tp_ffn_shard_workspace_bytes(2048, 8192, 16384, 1, B.TP_BF16) == \
        B.TP_FFN_NOALLOC_MAX_WORKSPACE
    assert lib.tp_ffn_shard_workspace_bytes(2048, 8192, 16448, 1, B.TP_BF16) > \
        B.TP_FFN_NOALLOC_MAX_WORKSPACE
    assert lib.tp_ffn_shard_workspace_bytes(2048, 64, 16384, 1, B.TP_BF16) == \
        B.TP_FFN_NOALLOC_MAX_WORKSPACE + 8 * 2048 * 64 * 4
    assert lib.tp_ffn_shard_workspace_bytes(1024, 16384, 22528, 1, B.TP_BF16) == \
        1024 * 22528 * 2 + 1024 * 16384 * 2 > B.TP_FFN_NOALLOC_MAX_WORKSPACE


def test_ffn_noalloc_zero_tokens_is_a_no_op(lib):
    st, msg = noalloc(lib, tokens=0, X=None, Y=None)
    assert st == 0, msg


def sp_call(lib, partials, R=None, x=None, y=Y, g=None, b=None, eps=1e-5, rows=64, cols=64,
            slice_=0, nslices=1, pdt=B.TP_BF16, rdt=B.TP_BF16, xdt=B.TP_F32, ydt=B.TP_BF16):
    arr = (ctypes.c_void_p * len(partials))(*partials)
    st = lib.tp_sp_reduce_layernorm(arr, len(partials), R, x, y, g, b, eps, rows, cols, slice_,
                                    nslices, pdt, rdt, xdt, ydt, None)
    return B.STATUS[st], lib.tp_last_error_message().decode()


def test_sp_reduce_layernorm_rejects(lib):
    assert sp_call(lib, [X, W1], pdt=9)[0] == "TP_ERR_DTYPE"
    assert sp_call(lib, [X, W1], x=WS, xdt=9)[0] == "TP_ERR_DTYPE"
    assert sp_call(lib, [])[0] == "TP_ERR_SHARD"
    assert sp_call(lib, [X], slice_=1, nslices=1)[0] == "TP_ERR_SHARD"
    assert sp_call(lib, [X], cols=60)[0] == "TP_ERR_SHAPE"            # not a multiple of 8
    assert sp_call(lib, [X], cols=32768 + 8)[0] == "TP_ERR_SHAPE"     # wider than a workgroup's row
    assert sp_call(lib, [X], eps=-1.0)[0] == "TP_ERR_SHAPE"
    assert sp_call(lib, [X], eps=float("nan"))[0] == "TP_ERR_SHAPE"
    assert sp_call(lib, [X, 0])[0] == "TP_ERR_NULL"
    assert sp_call(lib, [X], y=None)[0] == "TP_ERR_NULL"
    assert sp_call(lib, [X + 8])[0] == "TP_ERR_ALIGNMENT"
    assert sp_call(lib, [X], g=W2 + 4)[0] == "TP_ERR_ALIGNMENT"
    assert sp_call(lib, [X], y=X + 64)[0] == "TP_ERR_ALIAS"           # ln_out inside a partial
    assert sp_call(lib, [X], R=W1, y=W1)[0] == "TP_ERR_ALIAS"         # ln_out on the residual
    assert sp_call(lib, [X], x=Y + 16, y=Y)[0] == "TP_ERR_ALIAS"      # x_out overlaps ln_out
    assert sp_call(lib, [X], g=Y + 64, y=Y)[0] == "TP_ERR_ALIAS"      # gamma inside ln_out
    assert sp_call(lib, [X], x=X + 16)[0] == "TP_ERR_ALIAS"           # x_out partly over a partial


def test_sp_reduce_layernorm_empty_is_a_no_op(lib):
    assert sp_call(lib, [X], rows=0)[0] == "TP_SUCCESS"
    assert sp_call(lib, [X], rows=3, slice_=5, nslices=8)[0] == "TP_SUCCESS"   # empty block


def test_binding_refuses_tensors_on_another_device():
    """Every tensor of a call must sit on the device it runs on: the kernels
    would otherwise take another device's addresses as their own."""
    import torch
    from attention_shards_amd import binding as Bd
    a = torch.zeros(4)
    Bd._same_device(a.device, x=a, y=None)
    with pytest.raises(ValueError, match="W2_i is on cpu"):
        Bd._same_device(torch.device("cuda", 0), W2_i=a)
    assert Bd._nbytes(torch.zeros(5, dtype=torch.float32)) == 20
