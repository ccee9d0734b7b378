"""C-ABI contract checks that need no GPU: the library loads, exports every
declared call, and rejects invalid arguments before touching a device."""
import ctypes

import pytest

import long_context_attention_amd as sa
from long_context_attention_amd import _binding as B

FAKE = 0x100000          # aligned non-null stand-in pointer: never dereferenced on the error paths tested
MIS = 0x100004           # misaligned stand-in pointer


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def desc(**kw):
    base = dict(n_q_heads=4, n_kv_heads=1, head_dim=64, dtype=sa.SA_F32, rope_theta=1e4, softmax_scale=0.125)
    base.update(kw)
    return sa.make_desc(**base)


def test_exports_every_declared_symbol(lib):
    names = B.header_symbols()
    assert set(names) >= {"sa_phase1_encode", "sa_phase1_encode_anchor", "sa_phase1_encode_anchor_at",
                          "sa_anchor_at_workspace_bytes", "sa_decode_append", "sa_phase2_partial",
                          "sa_phase2_merge", "sa_workspace_bytes", "sa_last_error", "sa_abi_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_device_info_checks_its_pointers(lib):
    """sa_device_info refuses a NULL output, and without a GPU reports the runtime's error."""
    v = [ctypes.c_int32() for _ in range(4)]
    ptrs = [ctypes.byref(x) for x in v]
    assert lib_call("sa_device_info", None, *ptrs[1:]) == sa.SA_EINVAL
    rc = lib_call("sa_device_info", *ptrs)
    assert rc in (sa.SA_OK, sa.SA_EHIP)
    if rc == sa.SA_OK:
        assert v[0].value > 0 and v[1].value > 0


def test_last_error_is_per_thread(lib):
    """Two threads failing with different errors at the same time each read
    their own message (ctypes releases the interpreter lock during the call)."""
    import threading
    seen = {0: set(), 1: set()}

    def worker(k):
        for _ in range(300):
            if k == 0:
                assert _p1(desc(), L=1000, b=512) == sa.SA_EINVAL      # L % b != 0
            else:
                assert _p1(desc(), A=0) == sa.SA_EINVAL                # anchor out of range
            seen[k].add(sa.sa_last_error())

    ts = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert len(seen[0]) == 1 and len(seen[1]) == 1, seen
    assert seen[0] != seen[1]


def test_abi_version_and_desc_layout(lib):
    assert sa.sa_abi_version() == 1
    assert ctypes.sizeof(sa.sa_attn_desc) == 32


def _p1(d, L=2048, b=512, A=512, ptrs=(FAKE,) * 6):
    return lib_call("sa_phase1_encode", ctypes.byref(d) if d is not None else None, L, b, A, *ptrs, None, 0, None)


def lib_call(name, *args):
    return getattr(B.lib(), name)(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=3, n_kv_heads=2), sa.SA_EINVAL),
    (dict(head_dim=96), sa.SA_ENOTSUP),
    (dict(dtype=7), sa.SA_EINVAL),
    (dict(rope_theta=0.0), sa.SA_EINVAL),
    (dict(softmax_scale=float("nan")), sa.SA_EINVAL),
])
def test_phase1_rejects_bad_desc(lib, kw, code):
    assert _p1(desc(**kw)) == code
    assert sa.sa_last_error() != ""


def test_phase1_rejects_bad_sizes_and_pointers(lib):
    assert _p1(None) == sa.SA_EINVAL
    assert _p1(desc(), L=1000, b=512) == sa.SA_EINVAL                # L % b != 0
    assert "multiple" in sa.sa_last_error()
    assert _p1(desc(), L=(1 << 30) + 512, b=512) == sa.SA_EINVAL     # rows past 32-bit indexing
    assert "2^30" in sa.sa_last_error()
    assert _p1(desc(), A=513) == sa.SA_EINVAL                         # anchor longer than a block
    assert _p1(desc(), A=0) == sa.SA_EINVAL
    assert _p1(desc(), ptrs=(FAKE, FAKE, None, FAKE, FAKE, FAKE)) == sa.SA_EINVAL
    assert _p1(desc(), ptrs=(FAKE, FAKE, FAKE, MIS, FAKE, FAKE)) == sa.SA_EINVAL
    assert "aligned" in sa.sa_last_error()


def test_phase1_anchor_choice_is_checked(lib):
    def call(kind, A=512, ptrs=(FAKE,) * 6):
        return lib_call("sa_phase1_encode_anchor", ctypes.byref(desc()), 2048, 512, A, kind, *ptrs, None, 0, None)
    for kind in (2, -1, 7):
        assert call(kind) == sa.SA_EINVAL
        assert "anchor_kind" in sa.sa_last_error()
    for kind in (sa.SA_ANCHOR_FIRST, sa.SA_ANCHOR_PREVIOUS):   # the other checks are those of sa_phase1_encode
        assert call(kind, A=513) == sa.SA_EINVAL
        assert call(kind, ptrs=(FAKE, FAKE, FAKE, MIS, FAKE, FAKE)) == sa.SA_EINVAL


def test_phase1_anchor_positions_are_checked(lib):
    """sa_phase1_encode_anchor_at: every anchor inside its block's prefix, the
    workspace sized (n - 1) A Hkv d elements; all checked before any launch."""
    d = desc()                                             # f32, Hkv = 1, d = 64: L = 2048, b = 512, n = 4
    need = 3 * 200 * 1 * 64 * 4                            # the rotated keys (a multiple of 256 here)
    queues = sa.sa_workspace_bytes(sa.SA_CALL_PHASE1, d, 2048, 512, 1, 0)
    assert queues == 256                                   # the run-time job order's counters (optional)
    assert sa.sa_anchor_at_workspace_bytes(d, 2048, 512, 200) == need + queues
    assert sa.sa_anchor_at_workspace_bytes(desc(dtype=sa.SA_BF16, n_kv_heads=2, n_q_heads=4), 2048, 512, 512) == \
        3 * 512 * 2 * 64 * 2 + queues
    assert sa.sa_anchor_at_workspace_bytes(d, 512, 512, 512) == queues  # one block: no anchor keys
    assert sa.sa_anchor_at_workspace_bytes(d, 2048, 512, 513) == 0      # invalid arguments

    def call(pos, A=200, ws=FAKE, ws_bytes=need, ptrs=(FAKE,) * 6):
        arr = None if pos is None else (ctypes.c_int64 * len(pos))(*pos)
        return lib_call("sa_phase1_encode_anchor_at", ctypes.byref(d), 2048, 512, A, arr, *ptrs, ws, ws_bytes, None)
    assert call(None) == sa.SA_EINVAL and "anchor_pos" in sa.sa_last_error()
    for bad in ([0, 313, 0, 0], [0, 0, 825, 0], [0, 0, 0, -1]):          # block i's limit is (i-1) b - A
        assert call(bad) == sa.SA_EINVAL
        assert "anchor_pos" in sa.sa_last_error() and "prefix" in sa.sa_last_error()
    ok = [12345, 312, 824, 1336]                                         # entry 0 is ignored
    assert call(ok, ws_bytes=need - 1) == sa.SA_EWORKSPACE
    assert call(ok, ws=None) == sa.SA_EINVAL
    assert call(ok, ws=MIS) == sa.SA_EINVAL and "aligned" in sa.sa_last_error()
    assert call(ok, A=513) == sa.SA_EINVAL                               # sa_phase1_encode's own checks
    assert call(ok, ptrs=(FAKE, FAKE, FAKE, MIS, FAKE, FAKE)) == sa.SA_EINVAL


def test_append_rejects_tail_overflow(lib):
    d = desc()
    assert lib_call("sa_decode_append", ctypes.byref(d), FAKE, FAKE, 1, 0, FAKE, FAKE, (1 << 30) + 1, 0,
                    None) == sa.SA_EINVAL
    assert "2^30" in sa.sa_last_error()
    rc = lib.sa_decode_append(ctypes.byref(d), FAKE, FAKE, 5, 2048, FAKE, FAKE, 24, 20, None)
    assert rc == sa.SA_EINVAL and "overflow" in sa.sa_last_error()
    # sizes whose sum would overflow int64 are still a tail overflow
    rc = lib.sa_decode_append(ctypes.byref(d), FAKE, FAKE, 1 << 62, 2048, FAKE, FAKE, 24, 1 << 62, None)
    assert rc == sa.SA_EINVAL and "overflow" in sa.sa_last_error()
    # a grid past 2^32 work items is refused before any launch
    big = desc(n_q_heads=1 << 12, n_kv_heads=1 << 12, head_dim=128)
    rc = lib.sa_decode_append(ctypes.byref(big), FAKE, FAKE, 1 << 20, 0, FAKE, FAKE, 1 << 20, 0, None)
    assert rc == sa.SA_EINVAL and "too large" in sa.sa_last_error()
    assert lib.sa_decode_append(ctypes.byref(d), None, None, 0, 2048, None, None, 24, 3, None) == sa.SA_OK


def test_partial_workspace_contract(lib):
    d = desc()
    need = sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, d, 2048, 512, 16, 24)
    assert need > 0 and need % 4 == 0
    assert need == sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, d, 2048, 512, 16, 24)   # deterministic
    assert sa.sa_workspace_bytes(sa.SA_CALL_PHASE1, d, 2048, 512, 16, 24) == 256    # optional job counters
    assert sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, d, 2000, 512, 16, 24) == 0      # invalid sizes
    rc = lib.sa_phase2_partial(ctypes.byref(d), FAKE, 16, 2048, FAKE, FAKE, 2048, 512, FAKE, FAKE, 24, 16, 2048,
                               FAKE, FAKE, FAKE, need - 4, None)
    assert rc == sa.SA_EWORKSPACE
    rc = lib.sa_phase2_partial(ctypes.byref(d), FAKE, 16, 2048, FAKE, FAKE, 2048, 512, FAKE, FAKE, 24, 25, 2048,
                               FAKE, FAKE, FAKE, need, None)
    assert rc == sa.SA_EINVAL                                                        # tail_len > tail_cap


def test_step_rejects_bad_args(lib):
    d = desc()

    def call(t=1, tail_cap=24, tail_len=0, ws=(FAKE, 1 << 30), out=FAKE, kn=FAKE):
        return lib_call("sa_phase2_step", ctypes.byref(d), FAKE, kn, FAKE, t, FAKE, FAKE, 2048, 512, FAKE, FAKE,
                        tail_cap, tail_len, out, None, ws[0], ws[1], None)
    assert call(t=0) == sa.SA_EINVAL
    assert call(tail_len=24) == sa.SA_EINVAL                      # tail overflow
    assert "overflow" in sa.sa_last_error()
    assert call(kn=None) == sa.SA_EINVAL
    assert call(out=MIS) == sa.SA_EINVAL
    assert call(ws=(FAKE, 16)) == sa.SA_EWORKSPACE


def test_batched_decode_checks(lib):
    d = desc(dtype=sa.SA_BF16, n_q_heads=8, n_kv_heads=2, head_dim=128)
    assert ctypes.sizeof(sa.sa_decode_seq) == 104
    seq = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, k_tail=FAKE, v_tail=FAKE, out=FAKE,
               ctx_len=1024, block_len=256, tail_cap=8, tail_len=0)

    def call(seqs, n=None, dd=d, ws=1 << 30):
        arr = B.decode_seqs(seqs)
        return lib_call("sa_decode_step_batched", ctypes.byref(dd), len(seqs) if n is None else n, arr, FAKE, ws, None)
    assert B.sa_decode_batch_workspace_bytes(d, [seq] * 3) > 0
    assert call([seq] * 3, n=0) == sa.SA_EINVAL
    assert call([seq] * 3, n=sa.SA_MAX_BATCH + 1) == sa.SA_EINVAL
    assert call([seq], dd=desc(dtype=sa.SA_F32)) == sa.SA_ENOTSUP
    assert call([seq], dd=desc(dtype=sa.SA_BF16, n_q_heads=32, n_kv_heads=2, head_dim=128)) == sa.SA_ENOTSUP
    assert call([seq, seq, dict(seq, out=None)]) == sa.SA_EINVAL
    assert "sequence 2" in sa.sa_last_error()
    assert call([dict(seq, tail_len=8)]) == sa.SA_EINVAL              # no room for the new row
    assert call([dict(seq, ctx_len=1000)]) == sa.SA_EINVAL            # L % b != 0
    assert call([seq], ws=16) == sa.SA_EWORKSPACE


def test_merge_rejects_bad_args(lib):
    assert lib.sa_phase2_merge(0, 1, 4, 64, FAKE, FAKE, FAKE, sa.SA_F32, None, None) == sa.SA_EINVAL
    assert lib.sa_phase2_merge(5, 1, 4, 80, FAKE, FAKE, FAKE, sa.SA_F32, None, None) == sa.SA_ENOTSUP
    assert lib.sa_phase2_merge(5, 1, 4, 64, FAKE, FAKE, FAKE, 3, None, None) == sa.SA_EINVAL
    assert lib.sa_phase2_merge(5, 1, 4, 64, FAKE, FAKE, FAKE, sa.SA_F32, MIS, None) == sa.SA_EINVAL


def test_errors_raise_from_python_binding(lib):
    with pytest.raises(sa.StarAttnError) as e:
        sa.sa_phase1_encode(desc(), 1000, 512, 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0)
    assert e.value.code == sa.SA_EINVAL


def test_noalloc_step_checks(lib):
    """The no-allocation step checks its arguments like sa_phase2_step, and refuses
    a step whose workspace would not fit its fixed array before any device call."""
    d = desc()

    def call(t=1, tail_cap=24, tail_len=0, out=FAKE, kn=FAKE, L=2048, b=512, dd=d):
        return lib_call("sa_phase2_step_noalloc", ctypes.byref(dd), FAKE, kn, FAKE, t, FAKE, FAKE, L, b, FAKE, FAKE,
                        tail_cap, tail_len, out, None, None)
    assert call(t=0) == sa.SA_EINVAL
    assert call(tail_len=24) == sa.SA_EINVAL                      # tail overflow
    assert call(kn=None) == sa.SA_EINVAL
    assert call(out=MIS) == sa.SA_EINVAL
    assert call(L=2000) == sa.SA_EINVAL                           # ctx_len not a multiple of block_len
    big = desc(dtype=sa.SA_BF16, n_q_heads=64, n_kv_heads=8, head_dim=128)
    need = sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, big, 131072, 32768, 4096, 4096)
    assert need > sa.SA_NOALLOC_SCRATCH_BYTES
    assert call(t=4096, tail_cap=4096, L=131072, b=32768, dd=big) == sa.SA_EWORKSPACE
    assert "static array" in sa.sa_last_error()


def test_phase2_launch_sizes_are_bounded(lib):
    """Phase-2 calls whose launches would reach 2^32 work items are refused (no
    silent wrap of the grid size)."""
    d = desc(n_q_heads=1024, n_kv_heads=1024)

    def partial(t):
        return lib_call("sa_phase2_partial", ctypes.byref(d), FAKE, t, 2048, FAKE, FAKE, 2048, 512, FAKE, FAKE, 24, 0,
                        2048, FAKE, FAKE, FAKE, 1 << 62, None)
    assert partial((1 << 30) + 1) == sa.SA_EINVAL                 # t_q beyond 2^30
    assert partial(1 << 20) == sa.SA_EINVAL                       # 2^30 rows x 5 partitions
    assert "too large" in sa.sa_last_error()
    rc = lib_call("sa_phase2_merge", 5, 1 << 25, 1024, 64, FAKE, FAKE, FAKE, sa.SA_F32, None, None)
    assert rc == sa.SA_EINVAL and "too large" in sa.sa_last_error()
    assert lib_call("sa_phase2_merge", 0, 1, 1, 64, FAKE, FAKE, FAKE, sa.SA_F32, None, None) == sa.SA_EINVAL
