"""Host-side checks of the C-ABI library: exports, workspace sizing, the split
planner against the oracle's independent statement of it, and argument
validation.  No call here reaches a kernel launch (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from paged_gqa_decode_astr_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "astr_attn.h")).read()
    declared = set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(astr_\w+)\s*\(", header, re.M))
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    version = int(re.search(r"#define ASTR_ABI_VERSION (\d+)", header).group(1))
    assert lib.astr_abi_version() == version
    # Byte constants the binding mirrors.
    assert int(re.search(r"#define ASTR_WORKSPACE_COUNTER_BYTES (\d+)", header).group(1)) == _lib.WORKSPACE_COUNTER_BYTES
    m = re.search(r"#define ASTR_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", header)
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_workspace_size_formula(lib):
    for B, Hq, D, S in [(32, 32, 128, 0), (1, 4, 64, 7), (256, 32, 128, 64)]:
        cap = 256 if S == 0 else S
        P = cap + B - 1
        want = ((Hq * P * D * 4 + 255) // 256) * 256 + Hq * P * 8
        assert _lib.astr_workspace_size(B, Hq, D, S) == want
    assert _lib.astr_workspace_size(0, 32, 128, 0) == 0
    assert _lib.astr_workspace_size(4, 32, 128, -1) == 0


def _args(kv_indptr, Hq=32, Hkv=8, D=128, num_splits=0):
    a = _lib.PagedArgs()
    a.batch = len(kv_indptr) - 1
    a.num_qo_heads, a.num_kv_heads, a.head_dim = Hq, Hkv, D
    kvh = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    a.kv_indptr_host = kvh.ctypes.data_as(ctypes.c_void_p)
    a.num_splits = num_splits
    return a, kvh


def test_plan_matches_oracle_random():
    rng = np.random.default_rng(2024)
    for _ in range(3000):
        B = int(rng.integers(1, 300))
        hi = int(rng.choice([8, 64, 2000, 40000]))
        L = rng.integers(1, hi + 1, size=B)
        kv = np.concatenate([[0], np.cumsum(L)])
        Hkv = int(rng.choice([1, 2, 4, 8]))
        cus = int(rng.choice([1, 80, 256, 304]))
        D = int(rng.choice([32, 64, 128, 256]))
        a, keep = _args(kv, Hq=Hkv * 4, Hkv=Hkv, D=D)
        plan = _lib.astr_plan_decode(a, cus)
        want = oracle.plan_num_splits(kv, Hkv, cus, head_dim=D)
        assert plan.num_splits == want
        assert plan.num_partials == want + B - 1
        assert (plan.grid_x, plan.grid_y, plan.grid_z) == (want, Hkv, 1)
        assert plan.workspace_bytes == _lib.astr_workspace_size(B, Hkv * 4, D, want)


def test_plan_config_examples():
    from paged_gqa_decode_astr_amd.workloads import make_inputs
    for cid, want in [("tiny", None), ("decode_b32", 96)]:
        inp = make_inputs(cid, 0)
        a, keep = _args(inp["kv_indptr"], inp["num_qo_heads"], inp["num_kv_heads"], inp["head_dim"])
        plan = _lib.astr_plan_decode(a, 256)
        assert plan.num_splits == oracle.plan_num_splits(inp["kv_indptr"], inp["num_kv_heads"], 256)
        if want is not None:
            assert plan.num_splits == want


def test_plan_forced_and_errors():
    a, keep = _args([0, 5, 9], num_splits=3)
    assert _lib.astr_plan_decode(a, 256).num_splits == 3
    a.num_splits = -1
    with pytest.raises(_lib.AstrError) as ei:
        _lib.astr_plan_decode(a, 256)
    assert ei.value.status == _lib.ASTR_ERR_INVALID_ARG


# --------------------------------------------------------------------------- validation

FAKE = 0x10000  # 16-byte aligned stand-in for device pointers; never dereferenced on the host


def _valid_decode_args(kv=(0, 3, 7)):
    a, kvh = _args(list(kv), Hq=8, Hkv=2, D=64)
    a.sm_scale = 0.125
    for f in ("q", "o", "k_pool", "v_pool", "req_to_token", "kv_indptr"):
        setattr(a, f, FAKE)
    a.q_stride_tok, a.q_stride_head = 8 * 64, 64
    a.o_stride_tok, a.o_stride_head = 8 * 64, 64
    a.kv_stride_slot, a.kv_stride_head = 2 * 64, 64
    a.num_slots = 64
    a.req_to_token_stride = 8
    return a, kvh


def _call_decode(a, ws=FAKE, nbytes=1 << 30):
    lib = _lib.load_library()
    return lib.astr_paged_decode(ctypes.byref(a), ws, nbytes, None)


def _call_prefill(a):
    lib = _lib.load_library()
    return lib.astr_paged_prefill(ctypes.byref(a), None, 0, None)


@pytest.mark.parametrize("mutate,status,needle", [
    (lambda a: setattr(a, "q", None), 1, "q is NULL"),
    (lambda a: setattr(a, "kv_indptr_host", None), 1, "kv_indptr_host is NULL"),
    (lambda a: setattr(a, "num_kv_heads", 3), 1, "multiple"),
    (lambda a: setattr(a, "head_dim", 96), 2, "head_dim"),
    (lambda a: (setattr(a, "num_qo_heads", 32), setattr(a, "num_kv_heads", 2)), 2, "group"),
    (lambda a: setattr(a, "q", FAKE + 8), 1, "aligned"),
    (lambda a: setattr(a, "kv_stride_head", 60), 1, "kv_stride_head"),
    (lambda a: setattr(a, "o_stride_tok", 0), 1, "o_stride_tok"),
    (lambda a: setattr(a, "sm_scale", float("nan")), 1, "sm_scale"),
    (lambda a: setattr(a, "sm_scale", -0.125), 1, "sm_scale"),
    (lambda a: setattr(a, "sm_scale", 0.0), 1, "sm_scale"),
    (lambda a: setattr(a, "req_to_token_stride", 3), 1, "more than req_to_token_stride"),
    (lambda a: setattr(a, "num_slots", 0), 1, "num_slots"),
    (lambda a: setattr(a, "batch", -1), 1, "batch"),
    (lambda a: setattr(a, "qo_indptr", FAKE), 1, "no qo_indptr"),
    (lambda a: setattr(a, "num_splits", -2), 1, "num_splits"),
])
def test_decode_rejects_bad_arguments(mutate, status, needle):
    a, keep = _valid_decode_args()
    mutate(a)
    assert _call_decode(a) == status
    assert needle in _lib.astr_last_error()


@pytest.mark.parametrize("kv,needle", [((1, 3, 7), "kv_indptr[0]"), ((0, 3, 3), "seq_len must be >= 1"),
                                       ((0, 5, 2), "seq_len must be >= 1")])
def test_decode_rejects_bad_indptr(kv, needle):
    a, keep = _valid_decode_args(kv)
    assert _call_decode(a) == _lib.ASTR_ERR_INVALID_ARG
    assert needle in _lib.astr_last_error()


def test_decode_workspace_checks():
    a, keep = _valid_decode_args()
    a.num_splits = 4
    assert _call_decode(a, ws=None) == _lib.ASTR_ERR_WORKSPACE
    need = _lib.astr_workspace_size(2, 8, 64, 4)
    assert _call_decode(a, nbytes=need - 1) == _lib.ASTR_ERR_WORKSPACE
    assert "smaller" in _lib.astr_last_error()
    assert _call_decode(a, ws=FAKE + 4, nbytes=need) == _lib.ASTR_ERR_WORKSPACE


def test_empty_batch_is_a_noop():
    a, keep = _valid_decode_args((0,))
    assert _call_decode(a, ws=None, nbytes=0) == _lib.ASTR_OK
    a2, keep2 = _valid_decode_args((0,))
    assert _call_prefill(a2) == _lib.ASTR_OK


def _valid_prefill_args(kv=(0, 3, 7), qo=(0, 2, 3)):
    a, kvh = _valid_decode_args(kv)
    qoh = np.ascontiguousarray(qo, dtype=np.int32)
    a.qo_indptr = FAKE
    a.qo_indptr_host = qoh.ctypes.data_as(ctypes.c_void_p)
    return a, (kvh, qoh)


@pytest.mark.parametrize("qo,max_q,needle", [((0, 0, 3), 0, "q_len"), ((0, 4, 5), 0, "q_len"),
                                             ((1, 2, 3), 0, "qo_indptr[0]"), ((0, 2, 3), 1, "max_q_len")])
def test_prefill_rejects_bad_qlens(qo, max_q, needle):
    a, keep = _valid_prefill_args(qo=qo)
    a.max_q_len = max_q
    assert _call_prefill(a) == _lib.ASTR_ERR_INVALID_ARG
    assert needle in _lib.astr_last_error()


def test_prefill_needs_qo_indptr():
    a, keep = _valid_decode_args()
    assert _call_prefill(a) == _lib.ASTR_ERR_INVALID_ARG
    assert "qo_indptr" in _lib.astr_last_error()


# --------------------------------------------------------------------------- KV append validation

def _new_kv(k=FAKE, v=FAKE, stride_tok=2 * 64, stride_head=64):
    n = _lib.NewKV()
    n.k_new, n.v_new, n.stride_tok, n.stride_head = k, v, stride_tok, stride_head
    return n


def _call_append(a, n):
    lib = _lib.load_library()
    return lib.astr_kv_append(ctypes.byref(a), None if n is None else ctypes.byref(n), None)


def _call_decode_append(a, n, ws=FAKE, nbytes=1 << 30):
    lib = _lib.load_library()
    return lib.astr_paged_decode_append(ctypes.byref(a), None if n is None else ctypes.byref(n), ws, nbytes, None)


@pytest.mark.parametrize("mutate,needle", [
    (lambda a, n: setattr(n, "k_new", None), "k_new and v_new must be set"),
    (lambda a, n: setattr(n, "v_new", FAKE + 2), "aligned"),
    (lambda a, n: setattr(n, "stride_head", 12), "strides"),
    (lambda a, n: setattr(n, "stride_tok", 0), "strides"),
    (lambda a, n: setattr(a, "k_pool", None), "k_pool is NULL"),
    (lambda a, n: setattr(a, "head_dim", 60), "head_dim"),
    (lambda a, n: setattr(a, "kv_stride_slot", 100), "kv strides"),
    (lambda a, n: setattr(a, "num_slots", 0), "num_slots"),
    (lambda a, n: setattr(a, "req_to_token_stride", 3), "more than req_to_token_stride"),
    (lambda a, n: setattr(a, "qo_indptr", FAKE), "both be set"),
    (lambda a, n: setattr(a, "max_q_len", -1), "max_q_len"),
])
def test_append_rejects_bad_arguments(mutate, needle):
    a, keep = _valid_decode_args()
    n = _new_kv()
    mutate(a, n)
    assert _call_append(a, n) == _lib.ASTR_ERR_INVALID_ARG
    assert needle in _lib.astr_last_error()


@pytest.mark.parametrize("qo,max_q,needle", [((0, 0, 3), 0, "new tokens"), ((0, 4, 5), 0, "new tokens"),
                                             ((1, 2, 3), 0, "qo_indptr[0]"), ((0, 2, 3), 1, "max_q_len")])
def test_append_rejects_bad_new_counts(qo, max_q, needle):
    a, keep = _valid_prefill_args(qo=qo)
    a.max_q_len = max_q
    assert _call_append(a, _new_kv()) == _lib.ASTR_ERR_INVALID_ARG
    assert needle in _lib.astr_last_error()


def test_append_null_new_kv_and_empty_batch():
    a, keep = _valid_decode_args()
    assert _call_append(a, None) == _lib.ASTR_ERR_INVALID_ARG
    assert _call_decode_append(a, None) == _lib.ASTR_ERR_INVALID_ARG
    a0, keep0 = _valid_decode_args((0,))
    assert _call_append(a0, _new_kv()) == _lib.ASTR_OK
    assert _call_decode_append(a0, _new_kv(), ws=None, nbytes=0) == _lib.ASTR_OK


def test_decode_append_validates_like_decode():
    a, keep = _valid_decode_args()
    a.q = None
    assert _call_decode_append(a, _new_kv()) == _lib.ASTR_ERR_INVALID_ARG
    assert "q is NULL" in _lib.astr_last_error()
    a, keep = _valid_decode_args()
    assert _call_decode_append(a, _new_kv(stride_head=4)) == _lib.ASTR_ERR_INVALID_ARG
    a, keep = _valid_decode_args()
    a.num_splits = 4
    assert _call_decode_append(a, _new_kv(), ws=None) == _lib.ASTR_ERR_WORKSPACE


# --------------------------------------------------------------------------- decode graph validation

def _call_graph_create(layers, n, stream=FAKE, nkv=None):
    lib = _lib.load_library()
    out = ctypes.c_void_p(1234)
    st = lib.astr_decode_graph_create(layers, nkv, n, FAKE, 1 << 30, stream, ctypes.byref(out))
    return st, out


def test_graph_create_rejects_bad_arguments():
    arr = (_lib.PagedArgs * 2)()
    a0, k0 = _valid_decode_args()
    a1, k1 = _valid_decode_args()
    a0.num_splits = a1.num_splits = 4
    arr[0], arr[1] = a0, a1
    st, out = _call_graph_create(arr, 0)
    assert st == _lib.ASTR_ERR_INVALID_ARG and out.value is None
    st, out = _call_graph_create(arr, 2, stream=None)
    assert st == _lib.ASTR_ERR_INVALID_ARG and "non-null stream" in _lib.astr_last_error()
    arr[1].num_splits = 0
    st, out = _call_graph_create(arr, 2)
    assert st == _lib.ASTR_ERR_INVALID_ARG and "fixed plan" in _lib.astr_last_error()
    arr[1].num_splits = 4
    arr[1].batch = 1
    st, out = _call_graph_create(arr, 2)
    assert st == _lib.ASTR_ERR_INVALID_ARG and "one graph per batch size" in _lib.astr_last_error()
    lib = _lib.load_library()
    assert lib.astr_decode_graph_create(arr, None, 2, FAKE, 1 << 30, FAKE, None) == _lib.ASTR_ERR_INVALID_ARG
    assert lib.astr_decode_graph_launch(None, None) == _lib.ASTR_ERR_INVALID_ARG
    assert lib.astr_decode_graph_destroy(None) == _lib.ASTR_OK


# --------------------------------------------------------------------------- causal switch and mask validation

@pytest.mark.parametrize("setup,needle", [
    (lambda a: setattr(a, "non_causal", 2), "non_causal"),
    (lambda a: (setattr(a, "mask", FAKE + 2), setattr(a, "mask_stride_req", 8)), "multiples of 4"),
    (lambda a: (setattr(a, "mask", FAKE), setattr(a, "mask_stride_req", 6)), "multiples of 4"),
    (lambda a: (setattr(a, "mask", FAKE), setattr(a, "mask_stride_req", 4)), "mask rows hold 4"),
    (lambda a: (setattr(a, "mask", FAKE), setattr(a, "mask_stride_req", 8), setattr(a, "mask_stride_row", 4)),
     "mask rows hold 4"),
    (lambda a: (setattr(a, "mask", FAKE), setattr(a, "mask_stride_req", -4)), "mask strides"),
    (lambda a: (setattr(a, "mask", FAKE), setattr(a, "mask_stride_req", 1 << 32)), "mask strides"),
])
def test_decode_rejects_bad_mask(setup, needle):
    a, keep = _valid_decode_args((0, 3, 9))   # seq_lens 3 and 6
    setup(a)
    assert _call_decode(a) == _lib.ASTR_ERR_INVALID_ARG
    assert needle in _lib.astr_last_error()


def test_prefill_mask_needs_rows_for_every_query():
    a, keep = _valid_prefill_args(qo=(0, 2, 3))      # q_lens 2 and 1, seq_lens 3 and 4
    a.mask = FAKE
    a.mask_stride_row = 4
    a.mask_stride_req = 4                              # one row, but request 0 has two query rows
    assert _call_prefill(a) == _lib.ASTR_ERR_INVALID_ARG
    assert "query rows" in _lib.astr_last_error()


# --------------------------------------------------------------------------- page size validation

@pytest.mark.parametrize("ps,stride,kv,needle", [
    (3, 8, (0, 3, 7), "page_size"), (-2, 8, (0, 3, 7), "page_size"), (1 << 17, 8, (0, 3, 7), "page_size"),
    (4, 0, (0, 3, 7), "2-D page table"), (4, 1, (0, 3, 9), "table entries"),
])
def test_page_size_validation(ps, stride, kv, needle):
    """Rejected before any launch (only failing cases: a passing one would launch on placeholder pointers)."""
    a, keep = _valid_decode_args(kv)    # (0, 3, 9): a seq_len of 6 needs two pages of 4
    a.page_size = ps
    a.req_to_token_stride = stride
    assert _call_decode(a) == _lib.ASTR_ERR_INVALID_ARG
    assert needle in _lib.astr_last_error()


def _prefill_plan_args(qo, kv, Hq=32, Hkv=8, D=128, non_causal=False):
    a = _lib.PagedArgs()
    a.batch = len(kv) - 1
    a.num_qo_heads, a.num_kv_heads, a.head_dim = Hq, Hkv, D
    a.sm_scale = 0.1
    kvh = np.ascontiguousarray(kv, dtype=np.int32)
    qoh = np.ascontiguousarray(qo, dtype=np.int32)
    dummy = np.zeros(64, dtype=np.uint16)       # host memory: the planner never dereferences device pointers
    L = np.diff(kvh)
    a.q = a.o = a.k_pool = a.v_pool = ctypes.c_void_p(((dummy.ctypes.data + 15) // 16) * 16)
    a.q_stride_tok, a.q_stride_head = Hq * D, D
    a.o_stride_tok, a.o_stride_head = Hq * D, D
    a.kv_stride_slot, a.kv_stride_head = Hkv * D, D
    a.num_slots = int(kvh[-1]) + 1
    a.req_to_token = a.kv_indptr = a.qo_indptr = ctypes.c_void_p(dummy.ctypes.data)
    a.req_to_token_stride = int(L.max())
    a.kv_indptr_host = kvh.ctypes.data_as(ctypes.c_void_p)
    a.qo_indptr_host = qoh.ctypes.data_as(ctypes.c_void_p)
    a.non_causal = 1 if non_causal else 0
    return a, (kvh, qoh, dummy)


def test_prefill_plan_matches_oracle_random():
    """The library's automatic prefill plan equals the oracle's independent statement of it."""
    rng = np.random.default_rng(77)
    for _ in range(400):
        B = int(rng.integers(1, 120))
        hi = int(rng.choice([50, 2000, 40000]))
        L = rng.integers(1, hi + 1, size=B)
        q = np.array([int(rng.integers(1, min(int(x), int(rng.choice([8, 600]))) + 1)) for x in L])
        kv = np.concatenate([[0], np.cumsum(L)])
        qo = np.concatenate([[0], np.cumsum(q)])
        Hkv = int(rng.choice([1, 2, 4, 8, 16]))
        G = int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128, 256]))
        nc = bool(rng.integers(0, 2))
        cus = int(rng.choice([80, 256, 304]))
        a, keep = _prefill_plan_args(qo, kv, Hq=Hkv * G, Hkv=Hkv, D=D, non_causal=nc)
        got = _lib.astr_plan_prefill(a, cus)
        want, _ = oracle.prefill_plan(qo, kv, Hkv * G, Hkv, D, cus, non_causal=nc)
        if want is None:
            assert got.num_items == 0 and got.workspace_bytes == 0, B
            continue
        for f in ("num_items", "split_tiles", "chunk_tiles", "max_chunks", "partial_bytes", "workspace_bytes"):
            assert getattr(got, f) == want[f], (f, getattr(got, f), want[f], B, Hkv, G, D, nc, cus)


def test_prefill_plan_examples():
    # prefill_b8 seed 5000 on 256 CUs (512 slots): 448 whole tiles, so 64 items to spare.  Request 1
    # (seq_len 2301, q_len 316) has tiles of 32, 33, 33, 34, 34, ..., 36 key tiles; at T = 32 its
    # nine tiles above 32 would make 448 + 9 x 8 = 520 items, at T = 33 its seven tiles above 33
    # make 448 + 7 x 8 = 504, which fits: those seven are halved.
    from paged_gqa_decode_astr_amd.workloads import make_inputs
    inp = make_inputs("prefill_b8", 0)
    a, keep = _prefill_plan_args(inp["qo_indptr"], inp["kv_indptr"])
    p = _lib.astr_plan_prefill(a, 256)
    assert (p.num_items, p.split_tiles, p.chunk_tiles) == (504, 56, 33)
    # The same batch on 200 CUs (400 slots): the 448 whole tiles alone exceed them, nothing is split.
    p = _lib.astr_plan_prefill(a, 200)
    assert (p.num_items, p.split_tiles, p.workspace_bytes) == (448, 0, 0)
    # Two 20000-key requests with 64 new tokens: 16 tiles, each cut 16 ways.
    a, keep = _prefill_plan_args([0, 64, 128], [0, 20000, 40000])
    p = _lib.astr_plan_prefill(a, 256)
    assert (p.split_tiles, p.max_chunks, p.num_items) == (32, 16, 512)
