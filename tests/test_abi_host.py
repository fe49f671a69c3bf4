"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/qsa.h declares, and
reject every invalid argument before anything is enqueued (these calls never
reach the HIP runtime, so they run on a machine without a GPU).
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_trainable_amd as qsa
from block_sparse_trainable_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.library_path()):
        from block_sparse_trainable_amd import build
        build.build()
    return B.load()


def cfg(**kw):
    base = dict(block_size=4, token_budget=2048, idx_heads=4, idx_dim=128, rope_dims=64,
                q_heads=16, kv_heads=2, head_dim=128, dtype=B.QSA_BF16, rms_eps=1e-6,
                softmax_scale=0.0, rope_base=10000.0)
    base.update(kw)
    return B.QsaConfig(**base)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(B.EXPORTED) == set(names), names
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(qsa_[a-z_0-9]+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.qsa_abi_version() == 2


def test_config_struct_layout_matches_header():
    # int32 x 9, float x 2, double -> 9*4 + 2*4 = 44, padded to 48 for the double
    assert ctypes.sizeof(B.QsaConfig) == 56
    assert B.QsaConfig.rope_base.offset == 48


def test_status_strings(lib):
    for code, name in enumerate(["QSA_OK", "QSA_ERR_INVALID_ARGUMENT", "QSA_ERR_UNSUPPORTED",
                                 "QSA_ERR_WORKSPACE", "QSA_ERR_DEVICE"]):
        assert lib.qsa_status_string(code).decode() == name


def _al(v):
    return (v + 255) // 256 * 256


def test_workspace_sizes(lib):
    c = cfg()
    # select, many rows of at most 2^20 candidates: 16-bit score keys (64-row
    # tiles per sequence, rows padded to 64 blocks) and completion counters;
    # the rows are selected by streaming them, so no histograms
    rows, W = 2 * 8192, 34816
    want = _al(2 * rows * W)
    want = _al(want + 4 * rows)          # completion counters
    assert qsa.qsa_workspace_size(c, B.QSA_OP_SELECT, 2, 8192, 139264) == want
    # a ragged query count: each sequence's rows padded to a multiple of 64
    W = -(-((3000 - 1) // 4) // 64) * 64
    want = _al(2 * 2 * 3008 * W)
    want = _al(want + 4 * 2 * 3000)
    assert qsa.qsa_workspace_size(c, B.QSA_OP_SELECT, 2, 3000, 3000) == want
    # prefill rows of more than 2^20 candidates keep per-2048-block-segment
    # histograms (128 words)
    rows, c_max = 256, (4194310 - 1) // 4
    W = -(-c_max // 64) * 64
    nseg = -(-c_max // 2048)
    want = _al(4 * rows * W)
    want = _al(want + 4 * rows * nseg * 128)
    want = _al(want + 4 * rows)
    assert qsa.qsa_workspace_size(c, B.QSA_OP_SELECT, 1, 256, 4194310) == want
    # select, few long rows: 1024-block score segments and a row-wide
    # candidate array (4096 key/index pairs) for rows split over workgroups
    rows, c_max = 8, (262211 - 1) // 4
    W = -(-c_max // 4) * 4
    nseg = -(-c_max // 1024)
    want = _al(4 * rows * W)
    want = _al(want + 4 * rows * nseg * 128)
    want = _al(want + 8 * rows * 4096)
    want = _al(want + 4 * rows)
    assert qsa.qsa_workspace_size(c, B.QSA_OP_SELECT, 8, 1, 262211) == want
    assert qsa.qsa_workspace_size(c, B.QSA_OP_INDEX_BUILD, 1, 1, 10) == 0
    # prefill: a sort key and a walk start per row, and with 1,024 rows or
    # more an order slot
    assert qsa.qsa_workspace_size(c, B.QSA_OP_PREFILL, 1, 100, 100) == 8 * 100
    assert qsa.qsa_workspace_size(c, B.QSA_OP_PREFILL, 2, 8192, 139264) == 12 * 2 * 8192
    assert qsa.qsa_workspace_size(cfg(dtype=B.QSA_F32), B.QSA_OP_PREFILL, 2, 8192, 139264) == 0
    # decode: 17 splits of the token set, each 16 heads x (128 + 2) floats
    assert (qsa.qsa_workspace_size(c, B.QSA_OP_DECODE, 8, 1, 300000)
            == 4 * 8 * 17 * (16 * 128 + 32))
    assert qsa.qsa_workspace_size(cfg(dtype=B.QSA_F32), B.QSA_OP_DECODE, 8, 1, 300000) == 0


@pytest.mark.parametrize("field,value,status,word", [
    ("block_size", 6, B.QSA_ERR_UNSUPPORTED, "block_size"),     # not a power of two
    ("block_size", 3, B.QSA_ERR_UNSUPPORTED, "block_size"),
    ("block_size", 256, B.QSA_ERR_UNSUPPORTED, "block_size"),
    ("block_size", 0, B.QSA_ERR_INVALID_ARGUMENT, "positive"),
    ("idx_dim", 64, B.QSA_ERR_UNSUPPORTED, "idx_dim"),
    ("rope_dims", 62, B.QSA_ERR_UNSUPPORTED, "rope_dims"),
    ("head_dim", 96, B.QSA_ERR_UNSUPPORTED, "head_dim"),
    ("token_budget", 2052, B.QSA_ERR_UNSUPPORTED, "k_B"),      # k_B = 513 at r = 4
    ("kv_heads", 3, B.QSA_ERR_INVALID_ARGUMENT, "kv_heads"),
    ("dtype", 7, B.QSA_ERR_INVALID_ARGUMENT, "dtype"),
    ("rope_base", -1.0, B.QSA_ERR_INVALID_ARGUMENT, "rope_base"),
    ("rms_eps", -1.0, B.QSA_ERR_INVALID_ARGUMENT, "rms_eps"),
])
def test_config_validation(lib, field, value, status, word):
    c = cfg(**{field: value})
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_workspace_size(c, B.QSA_OP_SELECT, 1, 1, 8)
    assert e.value.status == status
    assert word in str(e.value)


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced


def test_block_sizes(lib):
    """r a power of two from 1 to 128 with k_B * r <= 2048 selected tokens
    (k_B <= 512 for r >= 4)."""
    for r in (1, 2, 4, 8, 16, 32, 64, 128):
        qsa.qsa_workspace_size(cfg(block_size=r), B.QSA_OP_SELECT, 1, 16, 4096)
    with pytest.raises(B.QsaError) as e:          # k_B = 2049 tokens
        qsa.qsa_workspace_size(cfg(block_size=1, token_budget=2049), B.QSA_OP_SELECT, 1, 1, 8)
    assert e.value.status == B.QSA_ERR_UNSUPPORTED and "2048" in str(e.value)
    # token level: r = 1, k_B = 2048 -> 2049 tokens; decode always keeps 17 splits
    assert (qsa.qsa_workspace_size(cfg(block_size=1), B.QSA_OP_DECODE, 2, 1, 300000)
            == 4 * 2 * 17 * (16 * 128 + 32))
    for op in (B.QSA_OP_BACKWARD, B.QSA_OP_DISTILL, B.QSA_OP_DECODE_STEP):
        with pytest.raises(B.QsaError) as e:      # built on 4-token units
            qsa.qsa_workspace_size(cfg(block_size=2), op, 1, 16, 4096)
        assert e.value.status == B.QSA_ERR_UNSUPPORTED
    with pytest.raises(B.QsaError) as e:          # k_B = 17 blocks of 128 = 2176 tokens
        qsa.qsa_workspace_size(cfg(block_size=128, token_budget=2049), B.QSA_OP_SELECT, 1, 1, 8)
    assert e.value.status == B.QSA_ERR_UNSUPPORTED and "2048" in str(e.value)
    # decode: 17 splits at every block size
    assert (qsa.qsa_workspace_size(cfg(block_size=16), B.QSA_OP_DECODE, 2, 1, 300000)
            == 4 * 2 * 17 * (16 * 128 + 32))
    assert (qsa.qsa_workspace_size(cfg(block_size=64, token_budget=512), B.QSA_OP_DECODE, 1, 1,
                                   300000) == 4 * 17 * (16 * 128 + 32))
    with pytest.raises(B.QsaError) as e:          # the fused step is built for r = 4 only
        qsa.qsa_decode_step(cfg(block_size=8), 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 4096,
                            FAKE, 4096, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30, stream=0)
    assert e.value.status == B.QSA_ERR_UNSUPPORTED and "block_size" in str(e.value)


def test_null_and_alignment_rejected_before_launch(lib):
    c = cfg()
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_index_build(c, 1, None, 64, FAKE, FAKE, 1, None, FAKE, stream=0)
    assert e.value.status == B.QSA_ERR_INVALID_ARGUMENT and "k_idx" in str(e.value)
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_select_topk(c, 1, 4, FAKE + 4, FAKE, 8, FAKE, 64, FAKE, FAKE, None, FAKE, 1 << 20,
                            stream=0)
    assert "q_idx" in str(e.value) and "16-byte" in str(e.value)
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_sparse_attn_prefill(c, 1, 4, FAKE, FAKE, FAKE, 64, FAKE, 8, FAKE, FAKE, None,
                                    None, None, 0, stream=0)
    assert "out" in str(e.value)


def test_sizes_rejected_before_launch(lib):
    c = cfg()
    for args, word in [((0, 4, 8), "batch"), ((1, 0, 8), "n_q"), ((1, 4, 0), "max_pos_end"),
                       ((1, 4, 65), "max_pos_end")]:
        b, nq, mpe = args
        with pytest.raises(B.QsaError) as e:
            qsa.qsa_sparse_attn_prefill(c, b, nq, FAKE, FAKE, FAKE, 64, FAKE, mpe, FAKE, FAKE, FAKE,
                                        None, None, 0, stream=0)
        assert e.value.status == B.QSA_ERR_INVALID_ARGUMENT and word in str(e.value)


def test_workspace_too_small_rejected(lib):
    c = cfg()
    need = qsa.qsa_workspace_size(c, B.QSA_OP_SELECT, 1, 16, 64)
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_select_topk(c, 1, 16, FAKE, FAKE, 64, FAKE, 64, FAKE, FAKE, None, FAKE, need - 1,
                            stream=0)
    assert e.value.status == B.QSA_ERR_WORKSPACE
    dneed = qsa.qsa_workspace_size(c, B.QSA_OP_DECODE, 2, 1, 64)
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_sparse_attn_decode(c, 2, FAKE, FAKE, FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE, None,
                                   None, dneed, stream=0)
    assert e.value.status == B.QSA_ERR_WORKSPACE


def test_product_has_no_oracle_dependency():
    pkg = os.path.join(ROOT, "block_sparse_trainable_amd")
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|from\s+\.\.oracle)|#include\s+.*oracle",
                     re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                assert not pat.search(open(os.path.join(dirpath, f)).read()), f


def test_decode_step_workspace_size(lib):
    c = cfg()
    # 3,325,952-byte control area, then (score, id) pairs of the score
    # segments (room for 1536 each: 1024 plus a remainder of up to 512),
    # per-segment suffix counts (128 words), 17 split states of 16 x (128 + 2)
    batch, mpe = 8, 262211
    c_max = (mpe - 1) // 4
    full, rem = divmod(c_max, 1024)
    nseg = full if rem <= 512 else full + 1
    # generation words, error word, split flags (32 per row), scoring flags
    # (264 per row), two buffers of 256 score-bin counts per row
    want = _al(4 * (4096 + 1024 * 32 + 1024 * 264 + 1024 * 2 * 256))
    assert want == 3325952 == B.QSA_STEP_CONTROL_BYTES
    want = _al(want + 8 * batch * nseg * 1536)
    want = _al(want + 4 * batch * nseg * 128)
    want = _al(want + 4 * batch * 17 * (16 * 128 + 32))
    assert nseg == 64
    assert qsa.qsa_workspace_size(c, B.QSA_OP_DECODE_STEP, batch, 1, mpe) == want


def _step(c, batch=2, mpe=64, ws_bytes=1 << 24, **ptr):
    p = dict(q_idx=FAKE, q=FAKE, k_idx=FAKE, k_cmp=FAKE, gain=None, k=FAKE, v=FAKE, pos=FAKE,
             sel=FAKE, cnt=FAKE, scs=None, out=FAKE, lse=None, ws=FAKE)
    p.update(ptr)
    qsa.qsa_decode_step(c, batch, p["q_idx"], p["q"], p["k_idx"], p["k_cmp"], p["gain"], p["k"],
                        p["v"], 1 << 21, p["pos"], mpe, p["sel"], p["cnt"], p["scs"], p["out"],
                        p["lse"], p["ws"], ws_bytes, stream=0)


@pytest.mark.parametrize("kw,args,status,word", [
    (dict(dtype=B.QSA_F32), {}, B.QSA_ERR_UNSUPPORTED, "bf16"),
    (dict(idx_heads=2), {}, B.QSA_ERR_UNSUPPORTED, "idx_heads"),
    (dict(q_heads=32, kv_heads=2), {}, B.QSA_ERR_UNSUPPORTED, "16 query heads"),
    ({}, dict(batch=1025), B.QSA_ERR_UNSUPPORTED, "batch"),
    ({}, dict(mpe=4 * 264192 + 5), B.QSA_ERR_UNSUPPORTED, "candidate blocks"),
    ({}, dict(ws_bytes=100), B.QSA_ERR_WORKSPACE, "workspace"),
    ({}, dict(q_idx=FAKE + 8), B.QSA_ERR_INVALID_ARGUMENT, "q_idx"),
    ({}, dict(k_cmp=None), B.QSA_ERR_INVALID_ARGUMENT, "k_cmp"),
    ({}, dict(pos=FAKE + 2), B.QSA_ERR_INVALID_ARGUMENT, "q_pos"),
])
def test_decode_step_rejects_before_launch(lib, kw, args, status, word):
    c = cfg(**kw)
    ptr = {k: v for k, v in args.items() if k not in ("batch", "mpe", "ws_bytes")}
    size = {k: v for k, v in args.items() if k in ("batch", "mpe", "ws_bytes")}
    with pytest.raises(B.QsaError) as e:
        _step(c, **size, **ptr)
    assert e.value.status == status
    assert word in str(e.value)


def test_backward_validation_and_workspace(lib):
    c = cfg(token_budget=256)                         # k_B = 64
    # MFMA shapes: counters per 16-token group, lists of uint2 (one per unit
    # of a largest token set, k_B + 1 at r = 4), D - D~ per head, q and dO
    # transposed, {P, weight} per (token of the set, head), and the row order
    # (sort key, walk start, order slot per row)
    ng = (1000 + 15) // 16
    want = _al(4 * 2 * ng)
    want = _al(want + 4 * 2 * ng)
    want = _al(want + 4 * (2 * ng + 1))
    want = _al(want + 8 * 1000 * 65)
    want = _al(want + 4 * 1000 * 16)
    want = _al(want + 2 * 1000 * 16 * 128)
    want = _al(want + 2 * 1000 * 16 * 128)
    want = _al(want + 8 * 1000 * 65 * 4 * 16)
    want = _al(want + 12 * 1000)
    assert qsa.qsa_workspace_size(c, B.QSA_OP_BACKWARD, 2, 500, 1000) == want
    # other shapes (fp32 here): per-block counters and lists, per-head D
    c32 = cfg(token_budget=256, dtype=B.QSA_F32, q_heads=4, kv_heads=1, head_dim=64)
    nb = (1000 + 3) // 4
    want = _al(4 * 2 * nb)
    want = _al(want + 4 * 2 * nb)
    want = _al(want + 4 * (2 * nb + 1))
    want = _al(want + 4 * 2 * 500 * 65)
    want = _al(want + 4 * 2 * 500 * 4)
    assert qsa.qsa_workspace_size(c32, B.QSA_OP_BACKWARD, 2, 500, 1000) == want
    args = [FAKE] * 3 + [1024, FAKE, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, 1 << 30]
    with pytest.raises(B.QsaError) as e:              # kv_heads > 2
        qsa.qsa_sparse_attn_backward(cfg(kv_heads=4), 1, 16, *args, stream=0)
    assert e.value.status == B.QSA_ERR_UNSUPPORTED and "kv_heads" in str(e.value)
    bad = list(args)
    bad[10] = None                                    # dout
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_sparse_attn_backward(c, 1, 16, *bad, stream=0)
    assert e.value.status == B.QSA_ERR_INVALID_ARGUMENT and "dout" in str(e.value)
    with pytest.raises(B.QsaError) as e:              # workspace too small
        qsa.qsa_sparse_attn_backward(c, 1, 16, *args[:-1], 64, stream=0)
    assert e.value.status == B.QSA_ERR_WORKSPACE


def test_offload_stage_validation(lib):
    c = cfg(token_budget=256)                           # k_B = 64: staging needs 65 * 4 tokens
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, 128, FAKE, FAKE]
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_offload_stage(c, 2, *args, 259, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.QSA_ERR_INVALID_ARGUMENT and "stage_tokens" in str(e.value)
    with pytest.raises(B.QsaError) as e:
        qsa.qsa_offload_stage(cfg(token_budget=256, dtype=B.QSA_F32), 2, *args, 260, FAKE, FAKE,
                              FAKE, FAKE, stream=0)
    assert e.value.status == B.QSA_ERR_UNSUPPORTED and "bf16" in str(e.value)
    with pytest.raises(B.QsaError) as e:                # hot_units
        bad = list(args)
        bad[9] = 0
        qsa.qsa_offload_stage(c, 2, *bad, 260, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.QSA_ERR_INVALID_ARGUMENT and "hot_units" in str(e.value)
