"""The C-ABI library: exports and host-side validation (CPU only, no compute
calls reach the GPU: every case here is rejected before any HIP call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")
LIB = os.environ.get("DSPARK_LIB_PATH") or os.path.join(ROOT, "semi_autoregressive_block_amd", "libdspark.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdspark.so is not built (run __graft_entry__.build())")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_dspark_lib", os.path.join(ROOT, "semi_autoregressive_block_amd", "_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod, mod.load(LIB)


def test_every_declared_symbol_is_exported(lib):
    mod, L = lib
    names = _declared()
    assert len(names) == 22, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mod.SIGNATURES)


def test_version_and_empty_error(lib):
    _, L = lib
    assert L.dspark_version() >= 100
    assert isinstance(L.dspark_last_error(), bytes)


def test_workspace_queries(lib):
    _, L = lib
    # attention needs one int32 launch-order slot per (request, tile, KV head)
    assert L.dspark_block_attention_workspace_bytes(128, 1, 16, 32, 8, 128, 8192) == 128 * 8 * 4
    assert L.dspark_block_attention_workspace_bytes(1, 512, 8, 32, 8, 128, 4096) == 256 * 8 * 4
    assert L.dspark_block_attention_workspace_bytes(1, 1, 1, 3, 2, 128, 10) == 0  # Hq % Hkv
    # gamma steps x 16 replica slots per row, each replica 4 KB-aligned
    assert L.dspark_markov_sample_workspace_bytes(64, 16, 151936, 256, 1) == 16 * 16 * 4096
    assert L.dspark_markov_sample_workspace_bytes(600, 2, 151936, 256, 1) == 2 * 16 * 8192
    # accept rate: one float share per (row, cluster member) + two 16-byte
    # statistics slots per member of every resident cluster + the error word;
    # V = 151936 bf16 is 18992 vectors per row, 768 per member -> G = 25
    G, rows = 25, 4 * 512 * 8
    assert L.dspark_accept_rate_workspace_bytes(4, 512, 8, 151936, 1) == \
        rows * G * 4 + (256 * 16 // G) * 2 * G * 16 + 64
    assert L.dspark_accept_rate_workspace_bytes(1, 1, 3, 1001, 1) == 0  # row-wise path


NULL = None


def test_attention_rejects_bad_arguments_before_any_hip_call(lib):
    mod, L = lib
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    def call(**kw):
        a = dict(B=1, A=1, gamma=8, Hq=4, Hkv=2, D=128, max_ctx=16, total_ctx=16, scale=0.1, dtype=1)
        a.update(kw)
        return L.dspark_block_attention(p, p, p, p, p, p, p, p, p, NULL, a["B"], a["A"], a["gamma"],
                                        a["Hq"], a["Hkv"], a["D"], a["max_ctx"], a["total_ctx"],
                                        a["scale"], a["dtype"], NULL, 0, NULL, NULL)
    assert call(D=96) == mod.ERR_INVALID_ARG and b"D must be" in L.dspark_last_error()
    assert call(Hq=3) == mod.ERR_INVALID_ARG
    assert call(gamma=65) == mod.ERR_INVALID_ARG
    assert call(dtype=7) == mod.ERR_INVALID_ARG
    assert call(scale=0.0) == mod.ERR_INVALID_ARG
    assert call(scale=float("nan")) == mod.ERR_INVALID_ARG
    assert call(B=-1) == mod.ERR_INVALID_ARG
    assert call(B=0) == mod.OK  # empty: nothing to do, nothing enqueued
    assert L.dspark_block_attention(NULL, p, p, p, p, p, p, p, p, NULL, 1, 1, 8, 4, 2, 128, 16, 16,
                                    0.1, 1, NULL, 0, NULL, NULL) == mod.ERR_INVALID_ARG


def test_markov_rejects_bad_arguments(lib):
    mod, L = lib
    p = ctypes.c_void_p(16)
    def call(R=4, gamma=2, V=64, r=8, wdtype=1, T=0.0, ws=p, wsb=1 << 20):
        return L.dspark_markov_sample(p, p, p, p, p, NULL, R, gamma, V, r, wdtype, T, 0, ws, wsb,
                                      NULL, NULL)
    assert call(r=0) == mod.ERR_INVALID_ARG
    assert call(r=2048) == mod.ERR_INVALID_ARG
    assert call(V=0) == mod.ERR_INVALID_ARG
    assert call(T=-1.0) == mod.ERR_INVALID_ARG
    assert call(T=float("inf")) == mod.ERR_INVALID_ARG
    assert call(wdtype=5) == mod.ERR_INVALID_ARG
    assert call(gamma=2000) == mod.ERR_INVALID_ARG
    assert call(wsb=8) == mod.ERR_WORKSPACE
    assert call(ws=NULL) == mod.ERR_WORKSPACE
    assert call(R=0) == mod.OK


def test_accept_rate_and_eval_mask_reject_bad_arguments(lib):
    mod, L = lib
    p = ctypes.c_void_p(16)
    assert L.dspark_accept_rate(p, p, p, NULL, NULL, 1, 1, 1, 1, 1, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_accept_rate(p, p, p, NULL, NULL, 1, 1, 1, 64, 3, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_accept_rate(p, p, p, NULL, NULL, 1, 1, 1, 64, 1, p, 0, NULL, NULL) == mod.ERR_WORKSPACE
    assert L.dspark_accept_rate(p, p, p, NULL, NULL, 0, 1, 1, 64, 1, NULL, 0, NULL, NULL) == mod.OK
    assert L.dspark_eval_mask(p, p, p, NULL, p, -1, 1, 1, 0, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_eval_mask(NULL, p, p, NULL, p, 1, 1, 1, 0, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_eval_mask(p, p, p, p, p, 1, 1, 1, 0, NULL, NULL) == mod.ERR_INVALID_ARG  # S_stride
    assert L.dspark_eval_mask(p, p, p, NULL, p, 0, 1, 1, 0, NULL, NULL) == mod.OK


def test_header_constants_match_binding(lib):
    """Every #define of the header has the same value in the Python binding."""
    mod, L = lib
    defs = dict(re.findall(r"#define\s+DSPARK_(\w+)\s+\(?(-?\d+)\)?", open(HEADER).read()))
    assert defs, "no constants parsed"
    for name, val in defs.items():
        assert getattr(mod, name) == int(val), name


def test_wait_limit_setter_is_host_only(lib):
    """Setting the poll limit touches no device; 0 restores the default."""
    _, L = lib
    L.dspark_set_wait_limit(5)
    L.dspark_set_wait_limit(0)


def test_block_logits_and_l1_loss_reject_bad_arguments(lib):
    mod, L = lib
    p = ctypes.c_void_p(16)
    # negative N, bad rank, unknown weight dtype, negative soft cap, missing workspace
    assert L.dspark_markov_block_logits(p, p, p, p, p, NULL, -1, 64, 8, 1, 0.0, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_block_logits(p, p, p, p, p, NULL, 4, 64, 0, 1, 0.0, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_block_logits(p, p, p, p, p, NULL, 4, 64, 8, 7, 0.0, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_block_logits(p, p, p, p, p, NULL, 4, 64, 8, 1, -1.0, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_block_logits(p, p, p, NULL, p, NULL, 4, 64, 8, 1, 0.0, p, 1 << 20, NULL, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_block_logits(p, p, p, p, p, NULL, 4, 64, 8, 1, 0.0, p, 0, NULL, NULL) == mod.ERR_WORKSPACE
    assert L.dspark_markov_block_logits(p, p, p, p, p, NULL, 0, 64, 8, 1, 0.0, NULL, 0, NULL, NULL) == mod.OK
    assert L.dspark_markov_block_logits_workspace_bytes(16384, 151936, 256, 1) == \
        L.dspark_markov_sample_workspace_bytes(16384, 1, 151936, 256, 1)
    # l1 loss: unknown dtype, bad decay, missing loss pointer, too small workspace
    assert L.dspark_l1_loss(p, p, NULL, 4.0, p, NULL, NULL, NULL, 1, 1, 1, 8, 3, p, 1 << 20, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_l1_loss(p, p, NULL, 0.0, p, NULL, NULL, NULL, 1, 1, 1, 8, 1, p, 1 << 20, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_l1_loss(p, p, NULL, 4.0, NULL, NULL, NULL, NULL, 1, 1, 1, 8, 1, p, 1 << 20, NULL) == mod.ERR_INVALID_ARG
    assert L.dspark_l1_loss(p, p, NULL, 4.0, p, NULL, NULL, NULL, 1, 1, 1, 8, 1, p, 0, NULL) == mod.ERR_WORKSPACE
    # rows that are not 16-byte vectors take the row-wise kernel: c | l1 | greedy only
    rows = 4 * 512 * 8
    assert L.dspark_l1_loss_workspace_bytes(4, 512, 8, 1001, 1) == 3 * rows * 4
    # clusters of 50 slices of 3072 elements (151936 / 3072 = 49.5): records [rows][50] of 16 bytes,
    # then statistics slots (2 x 50 x 16 bytes) and S slots (4 x 50 x 4 bytes) for at most
    # 4096 // 50 = 81 resident clusters, each part 256-byte aligned, and one 256-byte error word
    up = lambda x: (x + 255) // 256 * 256
    assert L.dspark_l1_loss_workspace_bytes(4, 512, 8, 151936, 1) == \
        3 * rows * 4 + rows * 50 * 16 + up(81 * 2 * 50 * 16) + up(81 * 4 * 50 * 4) + 256
    assert L.dspark_l1_loss_workspace_bytes(4, 512, 8, 151936, 3) == 0   # unknown dtype
    assert L.dspark_l1_loss_workspace_bytes(4, 512, 8, 0, 1) == 0


def test_confidence_schedule_rejects_bad_arguments(lib):
    mod, L = lib
    p = ctypes.c_void_p(16)
    args = lambda **k: dict(dict(hidden=p, hd=1, wh=p, bias=0.0, w1=NULL, wd=1, prev=NULL, we=NULL, r=0, V=0,
                                 sps=p, conf=NULL, surv=NULL, vlen=p, theta=NULL, B=1, A=1, g=4, H=8), **k)
    call = lambda a: L.dspark_confidence_schedule(a["hidden"], a["hd"], a["wh"], a["bias"], a["w1"], a["wd"],
                                                  a["prev"], a["we"], a["r"], a["V"], a["sps"], a["conf"],
                                                  a["surv"], a["vlen"], a["theta"], a["B"], a["A"], a["g"], a["H"],
                                                  NULL, NULL)
    assert call(args(g=2000)) == mod.ERR_INVALID_ARG              # gamma > 1024
    assert call(args(H=0)) == mod.ERR_INVALID_ARG
    assert call(args(hd=5)) == mod.ERR_INVALID_ARG
    assert call(args(we=p)) == mod.ERR_INVALID_ARG               # Markov input without w1 / prev
    assert call(args(bias=float("nan"))) == mod.ERR_INVALID_ARG
    assert call(args(vlen=NULL)) == mod.ERR_INVALID_ARG
    assert call(args(B=0)) == mod.OK


def test_head_workspaces_and_bad_arguments(lib):
    """Workspace sizes of the gated / recurrent heads and argument checks that
    return before any device work."""
    mod, L = lib
    # keys | P [splits][R*gamma, 3r] | E [R*gamma, r] | state [2, R, r], each 256-aligned.  The
    # projection's contraction is split so that at most 256 workgroups of 128x128 output tiles
    # run, at most 8 splits: 2048 x 768 is 96 tiles -> 2 splits, 2048 x 256 is 32 -> 8, 64 x 64 is 1 -> 8.
    R, g, r = 128, 16, 256
    keys = g * L.dspark_markov_sample_workspace_bytes(R, 1, 151936, r, 1)
    assert L.dspark_markov_head_sample_workspace_bytes(mod.HEAD_RNN, R, g, 151936, r) == \
        keys + 2 * R * g * 3 * r * 4 + R * g * r * 4 + 2 * R * r * 4
    assert L.dspark_markov_head_sample_workspace_bytes(mod.HEAD_GATED, R, g, 151936, r) == \
        keys + 8 * R * g * r * 4 + R * g * r * 4
    assert L.dspark_markov_head_sample_workspace_bytes(7, R, g, 151936, r) == 0
    assert L.dspark_markov_head_block_logits_workspace_bytes(mod.HEAD_GATED, 4, 16, 1000, 64) == \
        L.dspark_markov_block_logits_workspace_bytes(64, 1000, 64, 1) + 8 * 64 * 64 * 4 + 64 * 64 * 4
    null = None
    args = dict(kind=mod.HEAD_RNN, R=2, gamma=4, V=100, r=16, d=32, wdtype=1)

    def call(**kw):
        a = dict(args, **kw)
        return L.dspark_markov_head_sample(a["kind"], null, null, null, null, null, null, null, null, a["R"],
                                           a["gamma"], a["V"], a["r"], a["d"], a["wdtype"], 0.0, 0, null, 0,
                                           null, null)
    assert call(kind=0) == mod.ERR_INVALID_ARG
    assert call(r=12) == mod.ERR_INVALID_ARG          # rank not a multiple of 8
    assert call(r=520) == mod.ERR_INVALID_ARG         # rank above 512
    assert call(d=30) == mod.ERR_INVALID_ARG          # hidden size not a multiple of 8
    assert call(wdtype=5) == mod.ERR_INVALID_ARG
    assert call(gamma=1025) == mod.ERR_INVALID_ARG
    assert call() == mod.ERR_INVALID_ARG              # null pointers
    assert b"null required pointer" in L.dspark_last_error()
    assert call(R=0) == mod.OK                        # empty batch: nothing to do
    assert L.dspark_last_error() == b""
    rc = L.dspark_markov_head_block_logits(mod.HEAD_GATED, null, null, null, null, null, null, null, null, 2, 4,
                                           100, 16, 32, 1, -1.0, null, 0, null, null)
    assert rc == mod.ERR_INVALID_ARG                  # negative soft cap


def test_verify_workspace_and_bad_arguments(lib):
    mod, L = lib
    assert L.dspark_verify_workspace_bytes(128, 16) == 128 * 17 * 8 * 4 + 512 + 1024
    assert L.dspark_verify_workspace_bytes(0, 16) == 0
    n = None
    assert L.dspark_verify(n, n, n, n, n, 4, 2, 0, 1.0, 0, n, 0, n, n) == mod.ERR_INVALID_ARG      # V = 0
    assert L.dspark_verify(n, n, n, n, n, 4, 2, 10, -1.0, 0, n, 0, n, n) == mod.ERR_INVALID_ARG    # T < 0
    assert L.dspark_verify(n, n, n, n, n, 4, 2, 10, 1.0, 0, n, 0, n, n) == mod.ERR_INVALID_ARG     # null pointers
    assert L.dspark_verify(n, n, n, n, n, 0, 2, 10, 1.0, 0, n, 0, n, n) == mod.OK                  # nothing to do


def test_markov_noalloc_rejects_sizes_beyond_its_array(lib):
    mod, L = lib
    p = ctypes.c_void_p(1)
    # 128 rows x 65 steps of keys exceed the fixed array; refused on the host
    assert L.dspark_markov_sample_workspace_bytes(128, 65, 151936, 256, mod.BF16) > mod.NOALLOC_SCRATCH_BYTES
    rc = L.dspark_markov_sample_noalloc(p, p, p, p, p, None, 128, 65, 151936, 256, mod.BF16, 0.0, 0, None, None)
    assert rc == mod.ERR_WORKSPACE and b"above the fixed" in L.dspark_last_error()
    assert L.dspark_markov_sample_noalloc(None, p, p, p, p, None, 4, 2, 64, 32, mod.BF16, 0.0, 0, None,
                                          None) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_sample_noalloc(p, p, p, p, p, None, 4, 2, 64, 32, mod.BF16, -1.0, 0, None,
                                          None) == mod.ERR_INVALID_ARG
    assert L.dspark_markov_sample_noalloc(p, p, p, p, p, None, 0, 2, 64, 32, mod.BF16, 0.0, 0, None,
                                          None) == mod.OK


def test_noalloc_limit_matches_header(lib):
    mod, _ = lib
    src = open(HEADER).read()
    m = re.search(r"#define DSPARK_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and (int(m.group(1)) << int(m.group(2))) == mod.NOALLOC_SCRATCH_BYTES
