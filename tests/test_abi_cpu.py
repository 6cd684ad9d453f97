"""The C-ABI library loads and exports every entry point include/lola.h declares; host-side
validation answers without touching a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from hybrid_linear_attention_chunkwise_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lola.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:lola|hola)_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("liblola.so is not built (run __graft_entry__.build())")
    return B.load()


def test_header_declares_the_abi():
    assert _declared() == sorted(B.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (B.LOLA_OK, B.LOLA_EINVAL, B.LOLA_EUNSUPPORTED, B.LOLA_EDEVICE):
        assert B.status_string(code).startswith("LOLA_")
    assert "unknown" in B.status_string(42)


def _state(**kw):
    base = dict(B=2, n_heads=3, d_k=128, d_v=128, D=128, eta=256, lambda_=256, dtype=B.LOLA_BF16, t=0)
    base.update(kw)
    st = B.LolaState()
    for k, v in base.items():
        setattr(st, k, v)
    return st


def test_workspace_bytes_and_shape_checks(lib):
    st = _state()
    n1 = lib.lola_workspace_bytes(ctypes.byref(st), 4096, 64)
    n2 = lib.lola_workspace_bytes(ctypes.byref(st), 8192, 64)
    assert n1 > 0 and n2 > n1 and n1 % 256 == 0
    assert lib.lola_workspace_bytes(ctypes.byref(_state(d_k=96, d_v=96)), 64, 16) == 0
    assert lib.lola_workspace_bytes(ctypes.byref(_state(D=64)), 64, 16) == 0
    assert lib.lola_workspace_bytes(ctypes.byref(_state()), 64, 0) == 0
    assert lib.lola_workspace_bytes(ctypes.byref(_state(B=0)), 64, 16) == 0


def test_prefill_validation_without_gpu(lib):
    phi = B.LolaPhi(B.LOLA_PHI_SOFTMAX_PM, 128, 128, 0, None)
    st = _state()     # null device pointers
    rc = lib.lola_prefill(ctypes.byref(st), ctypes.byref(phi), None, None, None, 16, 16, None, None,
                          None, 0, None)
    assert rc == B.LOLA_EINVAL
    st = _state(d_k=96, d_v=96)
    rc = lib.lola_prefill(ctypes.byref(st), ctypes.byref(phi), None, None, None, 16, 16, None, None,
                          None, 0, None)
    assert rc == B.LOLA_EUNSUPPORTED
    rc = lib.lola_decode_step(ctypes.byref(_state()), ctypes.byref(phi), None, None, None, None, None, None)
    assert rc == B.LOLA_EINVAL
    rc = lib.lola_state_init(None, None)
    assert rc == B.LOLA_EINVAL


def _fake_ptrs(st):
    """Non-null, 256-byte aligned addresses that validation accepts (nothing reads them: every call
    below is rejected before any work is queued)."""
    for i, name in enumerate(("H", "s", "win_k", "win_v", "cache_k", "cache_v", "cache_pos")):
        setattr(st, name, 0x100000 + 0x1000 * i)
    return st


@pytest.mark.parametrize("mask,rule,reserved", [(0, 0, 0), (B.LOLA_READ_STATE | B.LOLA_READ_SPARSE, 0, 0),
                                                 (8 | B.LOLA_READ_WINDOW, 0, 0), (B.LOLA_READ_ALL, 5, 0),
                                                 (B.LOLA_READ_ALL, -1, 0), (B.LOLA_READ_ALL, 0, 1),
                                                 (B.LOLA_READ_ALL, 1, 0)])
def test_options_validation_without_gpu(lib, mask, rule, reserved):
    """Masks without the window or with other bits, unknown rules, non-zero reserved fields, and a
    query-accumulated rule on a state without score arrays are all rejected up front."""
    phi = B.LolaPhi(B.LOLA_PHI_SOFTMAX_PM, 128, 128, 0, 0x200000)
    st = _fake_ptrs(_state())
    opt = B.LolaOptions(mask, rule, 0, reserved)
    p = 0x300000
    rc = lib.lola_prefill_ex(ctypes.byref(st), ctypes.byref(phi), p, p, p, 16, 16, ctypes.byref(opt), p,
                             None, 0x400000, 1 << 40, None)
    assert rc == B.LOLA_EINVAL
    rc = lib.lola_decode_step_ex(ctypes.byref(st), ctypes.byref(phi), p, p, p, ctypes.byref(opt), p, None,
                                 None)
    assert rc == B.LOLA_EINVAL
    assert st.t == 0


HOLA_BAD = [
    # (B, heads, d, dtype, n, C, w, expected): rejected before any device work
    (0, 2, 128, B.LOLA_BF16, 64, 16, 4, B.LOLA_EINVAL),          # no sequences
    (1, 2, 96, B.LOLA_BF16, 64, 16, 4, B.LOLA_EUNSUPPORTED),     # d outside {64, 128, 256}
    (1, 2, 128, 7, 64, 16, 4, B.LOLA_EINVAL),                    # unknown storage type
    (1, 2, 128, B.LOLA_BF16, 64, 0, 4, B.LOLA_EINVAL),           # chunk of 0
    (1, 2, 128, B.LOLA_BF16, 64, 2048, 4, B.LOLA_EUNSUPPORTED),  # chunk above the largest
    (1, 2, 128, B.LOLA_BF16, -1, 16, 4, B.LOLA_EINVAL),          # negative length
    (1, 2, 128, B.LOLA_BF16, 64, 16, -1, B.LOLA_EINVAL),         # negative cache
    (1, 2, 128, B.LOLA_BF16, 64, 16, 65, B.LOLA_EUNSUPPORTED),   # cache above the largest
]


@pytest.mark.parametrize("Bn,h,d,dt,n,C,w,want", HOLA_BAD)
def test_hola_validation_without_gpu(lib, Bn, h, d, dt, n, C, w, want):
    """hola_prefill checks its shape arguments before touching memory; hola_workspace_bytes returns 0
    for a shape hola_prefill would reject."""
    p = 0x300000
    rc = lib.hola_prefill(Bn, h, d, dt, n, C, w, p, p, p, p, p, p, p, p, p, p, None, None, None, 0x400000, 1 << 40,
                          None)
    assert rc == want
    if w >= 0 and w <= 64:
        assert lib.hola_workspace_bytes(Bn, h, d, dt, n, C) == 0


def test_hola_pointer_validation_without_gpu(lib):
    """Null or misaligned tensors, and a workspace that is missing, misaligned or too small."""
    p = 0x300000
    good = dict(q=p, k=p, v=p, alpha=p, beta=p, gq=p, gk=p, sink=p, gate=p, y=p)
    need = lib.hola_workspace_bytes(1, 2, 128, B.LOLA_BF16, 64, 16)
    assert need > 0

    def call(ws=0x400000, nbytes=1 << 40, **over):
        a = dict(good, **over)
        return lib.hola_prefill(1, 2, 128, B.LOLA_BF16, 64, 16, 4, a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                a["gq"], a["gk"], a["sink"], a["gate"], a["y"], None, None, None, ws, nbytes, None)
    for name in good:
        assert call(**{name: None}) == B.LOLA_EINVAL, name
    for name in ("q", "k", "v", "y"):
        assert call(**{name: p + 2}) == B.LOLA_EINVAL, name
    assert call(ws=None) == B.LOLA_EINVAL
    assert call(ws=0x400010) == B.LOLA_EINVAL                       # workspace not 256-byte aligned
    assert call(nbytes=need - 1) == B.LOLA_EINVAL
    # an empty call is a no-op that needs no buffers at all
    assert lib.hola_prefill(1, 2, 128, B.LOLA_BF16, 0, 16, 4, None, None, None, None, None, None, None, None,
                            None, None, None, None, None, None, 0, None) == B.LOLA_OK


def _hola_state(**over):
    p = 0x300000
    f = dict(B=1, n_heads=2, d=128, dtype=B.LOLA_BF16, C=16, w=4, t=0, S=p, cache_pos=p, cache_score=p, cache_k=p,
             cache_v=p, open_k=p, open_v=p, open_score=p)
    f.update(over)
    return B.HolaState(*(f[name] for name, _ in B.HolaState._fields_))


def test_hola_state_validation_without_gpu(lib):
    """hola_state_init / hola_prefill_state / hola_decode_step reject a malformed state, a prefill from a
    non-empty memory and missing token arrays before anything is queued."""
    bad = [dict(d=96), dict(C=0), dict(C=2048), dict(w=-1), dict(w=65), dict(S=None), dict(open_k=None),
           dict(open_score=None), dict(open_v=0x300002), dict(cache_k=None), dict(cache_pos=None), dict(B=0)]
    want = [B.LOLA_EUNSUPPORTED, B.LOLA_EINVAL, B.LOLA_EUNSUPPORTED, B.LOLA_EINVAL, B.LOLA_EUNSUPPORTED,
            B.LOLA_EINVAL, B.LOLA_EINVAL, B.LOLA_EINVAL, B.LOLA_EINVAL, B.LOLA_EINVAL, B.LOLA_EINVAL, B.LOLA_EINVAL]
    for over, w_ in zip(bad, want):
        st = _hola_state(**over)
        assert lib.hola_state_init(ctypes.byref(st), None) == w_, over
    # w == 0 needs no cache arrays; a prefill needs an empty memory
    p = 0x300000
    st = _hola_state(w=0, cache_pos=None, cache_score=None, cache_k=None, cache_v=None, t=5)
    assert lib.hola_prefill_state(ctypes.byref(st), 64, p, p, p, p, p, p, p, p, p, p, 0x400000, 1 << 40,
                                  None) == B.LOLA_EUNSUPPORTED
    st = _hola_state()
    assert lib.hola_prefill_state(ctypes.byref(st), -1, p, p, p, p, p, p, p, p, p, p, 0x400000, 1 << 40,
                                  None) == B.LOLA_EINVAL
    assert lib.hola_prefill_state(ctypes.byref(st), 64, p, p, p, p, p, p, p, p, p, p, 0x400010, 1 << 40,
                                  None) == B.LOLA_EINVAL
    assert lib.hola_prefill_state(ctypes.byref(st), 0, None, None, None, None, None, None, None, None, None,
                                  None, None, 0, None) == B.LOLA_OK and st.t == 0
    args = [p] * 10
    for i in range(10):
        a = list(args)
        a[i] = None
        assert lib.hola_decode_step(ctypes.byref(st), *a, None) == B.LOLA_EINVAL, i
    assert st.t == 0


def test_overlap_validation_without_gpu(lib):
    """An overlap block needs a stream that is not the call's and all of its events; a bad block is
    rejected before anything is queued (the library owns no stream of its own to fall back on)."""
    phi = B.LolaPhi(B.LOLA_PHI_SOFTMAX_PM, 128, 128, 0, 0x200000)
    p = 0x300000
    good_events = [0x500000 + 0x100 * i for i in range(B.LOLA_OVERLAP_EVENTS)]
    cases = []
    for bad in range(B.LOLA_OVERLAP_EVENTS):
        ev = list(good_events)
        ev[bad] = 0
        cases.append((0x600000, ev, None))
    cases.append((0, good_events, None))              # no second stream
    cases.append((0x600000, good_events, 0x600000))   # the call's own stream
    for ov_stream, ev, call_stream in cases:
        st = _fake_ptrs(_state())
        ov = B.LolaOverlap(ov_stream, (ctypes.c_void_p * B.LOLA_OVERLAP_EVENTS)(*ev))
        opt = B.LolaOptions(B.LOLA_READ_ALL, 0, 0, 0, ctypes.pointer(ov))
        rc = lib.lola_prefill_ex(ctypes.byref(st), ctypes.byref(phi), p, p, p, 16, 16, ctypes.byref(opt), p,
                                 None, 0x400000, 1 << 40, call_stream)
        assert rc == B.LOLA_EINVAL
        assert st.t == 0


def test_no_process_wide_handles_in_the_sources():
    """The library keeps no stream, event, lock or cached device property between calls: no kernel
    source creates a stream or an event, holds a mutex, or caches a value in a static.  The one
    exception is the allocation-free entry point's scratch array and its per-device address
    (lola_noalloc.hip), which the header states."""
    csrc = os.path.join(ROOT, "hybrid_linear_attention_chunkwise_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "lola_noalloc.hip":
            continue
        text = open(os.path.join(csrc, name)).read()
        for banned in ("hipStreamCreate", "hipEventCreate", "std::mutex", "<mutex>"):
            assert banned not in text, (name, banned)
        for line in text.splitlines():
            code = line.split("//")[0].strip()
            if code.startswith("static ") and "=" in code and "constexpr" not in code and "(" not in code.split("=")[0]:
                raise AssertionError(f"{name}: static data: {line.strip()}")


def test_noalloc_rejects_before_any_work(lib):
    """lola_prefill_noalloc validates like lola_prefill_ex and refuses calls whose scratch exceeds its
    array (LOLA_NOALLOC_SCRATCH_BYTES) before touching the device."""
    phi = B.LolaPhi(B.LOLA_PHI_SOFTMAX_PM, 128, 128, 0, 0x200000)
    p = 0x300000
    st = _fake_ptrs(_state(d_k=96, d_v=96))
    assert lib.lola_prefill_noalloc(ctypes.byref(st), ctypes.byref(phi), p, p, p, 16, 16, None, p, None,
                                    None) == B.LOLA_EUNSUPPORTED
    st = _state()                                          # null state arrays
    assert lib.lola_prefill_noalloc(ctypes.byref(st), ctypes.byref(phi), p, p, p, 16, 16, None, p, None,
                                    None) == B.LOLA_EINVAL
    big = _fake_ptrs(_state(B=8, n_heads=32))
    n = 4096
    assert lib.lola_workspace_bytes(ctypes.byref(big), n, 64) > B.LOLA_NOALLOC_SCRATCH_BYTES
    assert lib.lola_prefill_noalloc(ctypes.byref(big), ctypes.byref(phi), p, p, p, n, 64, None, p, None,
                                    None) == B.LOLA_EUNSUPPORTED
    assert big.t == 0


def test_chunked_decode_validation_without_gpu(lib):
    """decode_chunk above 64, a chunked step with folded_pos, without the fold mask array, or with
    lambda > 0 and eta < decode_chunk - 1 are rejected before anything is queued."""
    phi = B.LolaPhi(B.LOLA_PHI_SOFTMAX_PM, 128, 128, 0, 0x200000)
    p = 0x300000
    cases = [(65, dict(), None), (8, dict(), 0x500000), (8, dict(dec_fold=0), None),
             (32, dict(eta=16), None)]
    for cd, over, folded in cases:
        st = _fake_ptrs(_state(eta=over.get("eta", 256)))
        st.dec_fold = over.get("dec_fold", 0x700000)
        opt = B.LolaOptions(B.LOLA_READ_ALL, 0, cd, 0, None)
        rc = lib.lola_decode_step_ex(ctypes.byref(st), ctypes.byref(phi), p, p, p, ctypes.byref(opt), p, folded,
                                     None)
        assert rc == B.LOLA_EINVAL, (cd, over)
        assert st.t == 0 and st.dec_chunk == 0
    st = _fake_ptrs(_state())
    st.dec_chunk = 8                      # a group is open: prefill is refused
    rc = lib.lola_prefill_ex(ctypes.byref(st), ctypes.byref(phi), p, p, p, 16, 16, None, p, None, 0x400000,
                             1 << 40, None)
    assert rc == B.LOLA_EINVAL
