"""CPU tests of the C ABI boundary (no GPU, no kernel launches).

The library must load, export every function that include/attn.h declares,
and reject bad arguments on the host with the documented status codes before
any HIP call.  Every call below violates at least one documented requirement,
so nothing is ever launched and the fake pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import tiled_exact_attention_flashattention_amd as tea
from tiled_exact_attention_flashattention_amd import (ATTN_BF16, ATTN_EINVAL, ATTN_EUNSUPPORTED,
                                                      ATTN_F32)

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == ["attn_bwd", "attn_bwd_workspace_size", "attn_decode_paged",
                                     "attn_decode_paged_fp8", "attn_decode_paged_int8",
                                     "attn_decode_paged_noalloc",
                                     "attn_decode_workspace_size",
                                     "attn_fwd", "attn_fwd_window", "attn_last_error",
                                     "attn_prefill_paged", "attn_status_string",
                                     "attn_time_next_call"]


def test_library_loads_and_exports_every_declared_symbol():
    L = tea.lib()
    raw = ctypes.CDLL(tea.library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name
        assert getattr(L, name) is not None


def test_status_strings():
    assert tea.attn_status_string(0) == "ATTN_OK"
    assert tea.attn_status_string(ATTN_EINVAL).startswith("ATTN_EINVAL")
    assert tea.attn_status_string(ATTN_EUNSUPPORTED).startswith("ATTN_EUNSUPPORTED")
    assert tea.attn_status_string(3).startswith("ATTN_EHIP")
    assert "unknown" in tea.attn_status_string(99)


def test_time_next_call_takes_both_events_or_neither():
    L = tea.lib()
    assert L.attn_time_next_call(None, None) == tea.ATTN_OK
    assert L.attn_time_next_call(ctypes.c_void_p(16), None) == ATTN_EINVAL
    assert tea.attn_last_error().startswith("attn_time_next_call")
    assert L.attn_time_next_call(None, ctypes.c_void_p(16)) == ATTN_EINVAL
    with pytest.raises(ValueError):
        class _Uncreated:
            cuda_event = 0
        tea.attn_time_next_call(_Uncreated(), _Uncreated())


def test_rejected_call_forgets_pending_timing_events():
    # A pair that is never a real event: if the rejected call kept it, the
    # next call would hand it to the HIP runtime.  Only host checks run here.
    L = tea.lib()
    assert L.attn_time_next_call(ctypes.c_void_p(16), ctypes.c_void_p(32)) == tea.ATTN_OK
    st = L.attn_fwd(None, None, None, None, None, 1, 1, 1, 1, 1, 64, 1.0, 0, 1, None)
    assert st == ATTN_EINVAL
    # cancelling is idempotent and succeeds whether or not a pair is pending
    assert L.attn_time_next_call(None, None) == tea.ATTN_OK


def _r256(x):
    return (x + 255) // 256 * 256


def _decode_ws(N, Hq, d):
    """Layout documented in include/attn.h: segment waves, partials, their LSEs."""
    waves, gmax = 768, 16
    return _r256(N * Hq * 8) + _r256(2 * waves * gmax * d * 4) + _r256(2 * waves * gmax * 4)


def test_workspace_size_formula():
    assert tea.attn_decode_workspace_size(64, 12, 128, 512, 16) == _decode_ws(64, 12, 128)
    assert tea.attn_decode_workspace_size(64, 12, 128, 512, 16) == 12687360
    assert tea.attn_decode_workspace_size(1, 1, 64, 1, 16) == _decode_ws(1, 1, 64)
    # independent of max_blocks (the split is decided on the device)
    assert tea.attn_decode_workspace_size(8, 4, 64, 7, 16) == tea.attn_decode_workspace_size(8, 4, 64, 9000, 16)
    assert tea.attn_decode_workspace_size(0, 12, 128, 512, 16) == 0
    assert tea.attn_decode_workspace_size(4, 12, 128, 512, 8) == 0


# --- attn_fwd argument checks --------------------------------------------------

P = 1 << 20     # fake, 16-byte aligned, never dereferenced
FWD_OK = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, B=1, Hq=4, Hkv=2, T=64, S=64, d=64,
              scale=0.125, causal=1, dtype=ATTN_BF16, stream=None)


def _fwd(**kw):
    a = dict(FWD_OK)
    a.update(kw)
    return tea.lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["T"], a["S"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), ATTN_EINVAL), (dict(k=None), ATTN_EINVAL), (dict(v=None), ATTN_EINVAL),
    (dict(o=None), ATTN_EINVAL),
    (dict(B=0), ATTN_EINVAL), (dict(Hq=0), ATTN_EINVAL), (dict(Hkv=0), ATTN_EINVAL),
    (dict(T=0), ATTN_EINVAL), (dict(S=0), ATTN_EINVAL), (dict(d=0), ATTN_EINVAL),
    (dict(T=-3), ATTN_EINVAL),
    (dict(Hq=5, Hkv=2), ATTN_EINVAL),
    (dict(T=65, S=64, causal=1), ATTN_EINVAL),
    (dict(scale=0.0), ATTN_EINVAL), (dict(scale=-0.1), ATTN_EINVAL),
    (dict(scale=float("nan")), ATTN_EINVAL), (dict(scale=float("inf")), ATTN_EINVAL),
    (dict(d=96), ATTN_EUNSUPPORTED), (dict(d=256), ATTN_EUNSUPPORTED), (dict(d=32), ATTN_EUNSUPPORTED),
    (dict(dtype=7), ATTN_EUNSUPPORTED),
    (dict(q=P + 8), ATTN_EINVAL), (dict(k=2 * P + 4), ATTN_EINVAL), (dict(o=4 * P + 2), ATTN_EINVAL),
    (dict(lse=5 * P + 2), ATTN_EINVAL),
    (dict(o=P), ATTN_EINVAL),                    # output aliases q
    (dict(lse=4 * P + 64), ATTN_EINVAL),         # lse inside o
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, T=1 << 12), ATTN_EINVAL),   # too large
])
def test_fwd_rejects_bad_arguments(bad, code):
    assert _fwd(**bad) == code
    assert tea.attn_last_error().startswith("attn_fwd")


def test_fwd_f32_shares_the_checks():
    assert _fwd(dtype=ATTN_F32, d=80) == ATTN_EUNSUPPORTED
    assert _fwd(dtype=ATTN_F32, T=100, S=50) == ATTN_EINVAL


def test_fwd_rejects_heads_past_32_bit_offsets():
    assert _fwd(T=1 << 24, S=1 << 24, d=128, B=1, Hq=1, Hkv=1, causal=0) == ATTN_EINVAL
    assert "2^31" in tea.attn_last_error()


def _fwd_window(window, **kw):
    a = dict(FWD_OK)
    a.update(kw)
    return tea.lib().attn_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                     a["Hkv"], a["T"], a["S"], a["d"], a["scale"], window,
                                     a["dtype"], a["stream"])


@pytest.mark.parametrize("window,bad,code", [
    (0, {}, ATTN_EINVAL), (-5, {}, ATTN_EINVAL),
    (16, dict(T=65, S=64), ATTN_EINVAL),          # causal needs T <= S
    (16, dict(q=None), ATTN_EINVAL), (16, dict(d=96), ATTN_EUNSUPPORTED),
    (16, dict(scale=float("nan")), ATTN_EINVAL), (16, dict(o=P), ATTN_EINVAL),
])
def test_fwd_window_rejects_bad_arguments(window, bad, code):
    assert _fwd_window(window, **bad) == code
    assert tea.attn_last_error().startswith("attn_fwd_window")


# --- attn_prefill_paged argument checks ------------------------------------------

PP_OK = dict(q=P, k=2 * P, v=3 * P, bt=4 * P, lens=5 * P, qlens=6 * P, o=7 * P, lse=8 * P, N=4,
             Hq=12, Hkv=2, T=64, d=128, page=16, num_pages=100, max_blocks=32, scale=0.088,
             window=0, dtype=ATTN_BF16, stream=None)


def _pp(**kw):
    a = dict(PP_OK)
    a.update(kw)
    return tea.lib().attn_prefill_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["qlens"],
                                        a["o"], a["lse"], a["N"], a["Hq"], a["Hkv"], a["T"],
                                        a["d"], a["page"], a["num_pages"], a["max_blocks"],
                                        a["scale"], a["window"], a["dtype"], a["stream"])


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), ATTN_EINVAL), (dict(bt=None), ATTN_EINVAL), (dict(qlens=None), ATTN_EINVAL),
    (dict(o=None), ATTN_EINVAL),
    (dict(N=0), ATTN_EINVAL), (dict(T=0), ATTN_EINVAL), (dict(num_pages=0), ATTN_EINVAL),
    (dict(max_blocks=0), ATTN_EINVAL), (dict(Hq=12, Hkv=5), ATTN_EINVAL),
    (dict(window=-1), ATTN_EINVAL), (dict(scale=0.0), ATTN_EINVAL),
    (dict(dtype=ATTN_F32), ATTN_EUNSUPPORTED), (dict(page=32), ATTN_EUNSUPPORTED),
    (dict(d=96), ATTN_EUNSUPPORTED),
    (dict(q=P + 4), ATTN_EINVAL), (dict(qlens=6 * P + 2), ATTN_EINVAL),
    (dict(o=P), ATTN_EINVAL),                   # output aliases q
    (dict(lse=7 * P + 256), ATTN_EINVAL),       # lse inside o
    (dict(o=5 * P), ATTN_EINVAL),               # output over seq_lens
])
def test_prefill_paged_rejects_bad_arguments(bad, code):
    assert _pp(**bad) == code
    assert tea.attn_last_error().startswith("attn_prefill_paged")


# --- attn_bwd argument checks ---------------------------------------------------

def _bwd_ws(B, Hq, Hkv, T, S, d):
    """Layout documented in include/attn.h: row statistics, then head-split partials."""
    hpg, base = Hq // Hkv, -(-S // 128) * B * Hkv
    n = next((m for m in range(1, hpg + 1) if hpg % m == 0 and base * m >= 512), hpg)
    return _r256(B * Hq * T * 8) + (2 * n * B * Hkv * S * d * 4 if n > 1 else 0)


def test_bwd_workspace_size_formula():
    assert tea.attn_bwd_workspace_size(4, 12, 2, 4096, 4096, 128) == 68681728   # 2 head splits
    assert tea.attn_bwd_workspace_size(8, 12, 12, 1024, 1024, 64) == 786432      # no split
    for args in [(4, 12, 2, 4096, 4096, 128), (8, 12, 12, 1024, 1024, 64), (1, 1, 1, 1, 1, 64),
                 (1, 32, 4, 100, 100, 128), (2, 12, 4, 777, 1500, 64), (3, 6, 1, 10, 3000, 128)]:
        assert tea.attn_bwd_workspace_size(*args) == _bwd_ws(*args), args
    assert tea.attn_bwd_workspace_size(1, 1, 1, 1, 1, 64) == 256
    assert tea.attn_bwd_workspace_size(0, 1, 1, 1, 1, 64) == 0
    assert tea.attn_bwd_workspace_size(1, 1, 1, 0, 1, 64) == 0
    assert tea.attn_bwd_workspace_size(1, 6, 4, 8, 8, 64) == 0      # Hq not a multiple of Hkv


BWD_WS = tea.attn_bwd_workspace_size(1, 4, 2, 64, 64, 64)
BWD_OK = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, do=6 * P, dq=7 * P, dk=8 * P, dv=9 * P,
              B=1, Hq=4, Hkv=2, T=64, S=64, d=64, scale=0.125, causal=1, dtype=ATTN_BF16,
              ws=10 * P, ws_bytes=BWD_WS, stream=None)


def _bwd(**kw):
    a = dict(BWD_OK)
    a.update(kw)
    return tea.lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                              a["dv"], a["B"], a["Hq"], a["Hkv"], a["T"], a["S"], a["d"], a["scale"],
                              a["causal"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), ATTN_EINVAL), (dict(lse=None), ATTN_EINVAL), (dict(do=None), ATTN_EINVAL),
    (dict(dq=None), ATTN_EINVAL), (dict(dk=None), ATTN_EINVAL), (dict(dv=None), ATTN_EINVAL),
    (dict(ws=None), ATTN_EINVAL),
    (dict(B=0), ATTN_EINVAL), (dict(T=0), ATTN_EINVAL), (dict(S=0), ATTN_EINVAL),
    (dict(Hq=6, Hkv=4), ATTN_EINVAL),
    (dict(T=65, S=64, causal=1), ATTN_EINVAL),
    (dict(scale=0.0), ATTN_EINVAL), (dict(scale=float("nan")), ATTN_EINVAL),
    (dict(dtype=ATTN_F32), ATTN_EUNSUPPORTED), (dict(dtype=9), ATTN_EUNSUPPORTED),
    (dict(d=96), ATTN_EUNSUPPORTED),
    (dict(do=6 * P + 8), ATTN_EINVAL), (dict(dk=8 * P + 2), ATTN_EINVAL),
    (dict(lse=5 * P + 2), ATTN_EINVAL), (dict(ws=10 * P + 4), ATTN_EINVAL),
    (dict(ws_bytes=BWD_WS - 1), ATTN_EINVAL),
    (dict(dq=P), ATTN_EINVAL),                   # dq aliases q
    (dict(dv=6 * P + 256), ATTN_EINVAL),         # dv inside dO
    (dict(dk=7 * P + 512), ATTN_EINVAL),         # dk inside dq
    (dict(ws=9 * P), ATTN_EINVAL),               # workspace aliases dv
    (dict(T=1 << 24, S=1 << 24, d=128, causal=0, ws_bytes=1 << 40), ATTN_EINVAL),   # 32-bit offsets
])
def test_bwd_rejects_bad_arguments(bad, code):
    assert _bwd(**bad) == code
    assert tea.attn_last_error().startswith("attn_bwd")


# --- attn_decode_paged argument checks ------------------------------------------

WS = tea.attn_decode_workspace_size(8, 12, 128, 64, 16)
DEC_OK = dict(q=P, k=2 * P, v=3 * P, bt=4 * P, lens=5 * P, o=6 * P, lse=7 * P, N=8, Hq=12, Hkv=2,
              d=128, page=16, num_pages=100, max_blocks=64, scale=0.088, dtype=ATTN_BF16,
              ws=8 * P, ws_bytes=WS, stream=None)


def _dec(**kw):
    a = dict(DEC_OK)
    a.update(kw)
    return tea.lib().attn_decode_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["o"], a["lse"],
                                       a["N"], a["Hq"], a["Hkv"], a["d"], a["page"], a["num_pages"],
                                       a["max_blocks"], a["scale"], a["dtype"], a["ws"],
                                       a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), ATTN_EINVAL), (dict(k=None), ATTN_EINVAL), (dict(v=None), ATTN_EINVAL),
    (dict(bt=None), ATTN_EINVAL), (dict(lens=None), ATTN_EINVAL), (dict(o=None), ATTN_EINVAL),
    (dict(N=0), ATTN_EINVAL), (dict(Hq=0), ATTN_EINVAL), (dict(Hkv=0), ATTN_EINVAL),
    (dict(num_pages=0), ATTN_EINVAL), (dict(max_blocks=0), ATTN_EINVAL),
    (dict(Hq=12, Hkv=5), ATTN_EINVAL),
    (dict(scale=0.0), ATTN_EINVAL), (dict(scale=float("nan")), ATTN_EINVAL),
    (dict(dtype=ATTN_F32), ATTN_EUNSUPPORTED), (dict(page=8), ATTN_EUNSUPPORTED),
    (dict(page=32), ATTN_EUNSUPPORTED), (dict(d=96), ATTN_EUNSUPPORTED),
    (dict(Hq=34, Hkv=2), ATTN_EUNSUPPORTED),
    (dict(q=P + 4), ATTN_EINVAL), (dict(bt=4 * P + 2), ATTN_EINVAL),
    (dict(ws=None), ATTN_EINVAL), (dict(ws_bytes=WS - 1), ATTN_EINVAL), (dict(ws=8 * P + 8), ATTN_EINVAL),
    (dict(N=4096, Hkv=12, Hq=12, max_blocks=1 << 17, ws_bytes=1 << 40), ATTN_EINVAL),   # > 2^31 pairs
    (dict(o=P), ATTN_EINVAL),                    # output aliases q
    (dict(o=5 * P), ATTN_EINVAL),                # output over seq_lens
    (dict(lse=4 * P + 64), ATTN_EINVAL),         # lse inside the block table
    (dict(lse=6 * P + 64), ATTN_EINVAL),         # lse inside o
    (dict(ws=2 * P), ATTN_EINVAL),               # workspace over the key pool
    (dict(ws=6 * P - 1024), ATTN_EINVAL),        # workspace runs into o
    (dict(o=8 * P + 4096), ATTN_EINVAL),         # o inside the workspace
])
def test_decode_rejects_bad_arguments(bad, code):
    assert _dec(**bad) == code
    assert tea.attn_last_error().startswith("attn_decode_paged")


def _dec_na(**kw):
    a = dict(DEC_OK)
    a.update(kw)
    return tea.lib().attn_decode_paged_noalloc(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["o"],
                                               a["lse"], a["N"], a["Hq"], a["Hkv"], a["d"],
                                               a["page"], a["num_pages"], a["max_blocks"],
                                               a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), ATTN_EINVAL), (dict(lens=None), ATTN_EINVAL), (dict(N=0), ATTN_EINVAL),
    (dict(Hq=12, Hkv=5), ATTN_EINVAL), (dict(scale=float("nan")), ATTN_EINVAL),
    (dict(dtype=ATTN_F32), ATTN_EUNSUPPORTED), (dict(page=32), ATTN_EUNSUPPORTED),
    (dict(d=96), ATTN_EUNSUPPORTED), (dict(q=P + 4), ATTN_EINVAL),
    (dict(o=P), ATTN_EINVAL), (dict(lse=6 * P + 64), ATTN_EINVAL),
    (dict(N=5462, Hq=12, Hkv=2), ATTN_EINVAL),      # N*Hq = 65544 rows: more than the scratch holds
    (dict(N=65535, Hq=16, Hkv=16), ATTN_EINVAL),
])
def test_decode_noalloc_rejects_bad_arguments(bad, code):
    assert _dec_na(**bad) == code
    assert tea.attn_last_error().startswith("attn_decode_paged_noalloc")


def test_decode_noalloc_names_the_scratch_limit():
    assert _dec_na(N=5462, Hq=12, Hkv=2) == ATTN_EINVAL
    assert "scratch" in tea.attn_last_error() and "65536" in tea.attn_last_error()


def _dec8(k_scale=0.03, v_scale=0.03, **kw):
    a = dict(DEC_OK)
    a.update(kw)
    return tea.lib().attn_decode_paged_fp8(a["q"], a["k"], a["v"], k_scale, v_scale, a["bt"],
                                           a["lens"], a["o"], a["lse"], a["N"], a["Hq"], a["Hkv"],
                                           a["d"], a["page"], a["num_pages"], a["max_blocks"],
                                           a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("scales,bad,code", [
    ((0.0, 0.03), {}, ATTN_EINVAL), ((0.03, -1.0), {}, ATTN_EINVAL),
    ((float("nan"), 0.03), {}, ATTN_EINVAL), ((0.03, float("inf")), {}, ATTN_EINVAL),
    ((1e38, 0.03), dict(scale=1e3), ATTN_EINVAL),          # scale * k_scale overflows
    ((0.03, 0.03), dict(q=None), ATTN_EINVAL), ((0.03, 0.03), dict(page=8), ATTN_EUNSUPPORTED),
    ((0.03, 0.03), dict(d=96), ATTN_EUNSUPPORTED), ((0.03, 0.03), dict(ws_bytes=WS - 1), ATTN_EINVAL),
    ((0.03, 0.03), dict(k=2 * P + 8), ATTN_EINVAL), ((0.03, 0.03), dict(Hq=34, Hkv=2), ATTN_EUNSUPPORTED),
    ((0.03, 0.03), dict(ws=3 * P), ATTN_EINVAL),             # workspace over the value pool
    ((0.03, 0.03), dict(lse=P + 16), ATTN_EINVAL),           # lse inside q
])
def test_decode_fp8_rejects_bad_arguments(scales, bad, code):
    assert _dec8(*scales, **bad) == code
    assert tea.attn_last_error().startswith("attn_decode_paged_fp8")


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tea.attn_fwd(q, q, q, torch.empty_like(q), None, 0.125, False)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import tiled_exact_attention_flashattention_amd._binding as b
    monkeypatch.setattr(b, "_LIB", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "libattn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        b.lib()


def test_one_hip_runtime_per_process():
    """libattn.so must bind to torch's HIP runtime, never map a second one."""
    import tiled_exact_attention_flashattention_amd._binding as b
    tea.lib()
    assert len(b.hip_runtimes_loaded()) == 1, b.hip_runtimes_loaded()


_EHIP_CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
if torch.cuda.device_count() != 0:      # a visible device: never call with fake pointers
    print("DEVICE_VISIBLE")
    sys.exit(0)
import tiled_exact_attention_flashattention_amd as tea
L = tea.lib()
P = 1 << 20
out = []
# arguments that pass every host check, so the call reaches the HIP launch
out.append(L.attn_fwd(P, 2 * P, 3 * P, 4 * P, 5 * P, 1, 4, 2, 64, 64, 64, 0.125, 1, 1, None))
out.append(tea.attn_last_error())
ws = tea.attn_decode_workspace_size(8, 12, 128, 64, 16)
out.append(L.attn_decode_paged(P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8, 12, 2, 128, 16, 100,
                               64, 0.088, 1, 8 * P, ws, None))
out.append(tea.attn_last_error())
print(repr(out))
"""


def test_hip_failure_surfaces_as_ehip():
    """With no device visible to HIP, a call whose arguments pass every host
    check fails at the launch: it must return ATTN_EHIP with the runtime's
    message, never crash or fall back.  Run in a child process whose HIP sees
    no device, so nothing reaches a GPU even on a GPU host."""
    import subprocess
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="99", ROCR_VISIBLE_DEVICES="99",
               CUDA_VISIBLE_DEVICES="99")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _EHIP_CHILD, root], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    if r.stdout.strip().endswith("DEVICE_VISIBLE"):
        pytest.skip("HIP still sees a device with HIP_VISIBLE_DEVICES=99")
    import ast
    fwd_rc, fwd_msg, dec_rc, dec_msg = ast.literal_eval(r.stdout.strip().splitlines()[-1])
    assert fwd_rc == 3 and fwd_msg.startswith("attn_fwd: "), (fwd_rc, fwd_msg)
    assert dec_rc == 3 and dec_msg.startswith("attn_decode_paged: "), (dec_rc, dec_msg)


def _dec_i8(k_scale=0.03, v_scale=0.03, **kw):
    a = dict(DEC_OK)
    a.update(kw)
    return tea.lib().attn_decode_paged_int8(a["q"], a["k"], a["v"], k_scale, v_scale, a["bt"],
                                            a["lens"], a["o"], a["lse"], a["N"], a["Hq"], a["Hkv"],
                                            a["d"], a["page"], a["num_pages"], a["max_blocks"],
                                            a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("scales,bad,code", [
    ((0.0, 0.03), {}, ATTN_EINVAL), ((0.03, -1.0), {}, ATTN_EINVAL),
    ((float("nan"), 0.03), {}, ATTN_EINVAL), ((0.03, float("inf")), {}, ATTN_EINVAL),
    ((1e38, 0.03), dict(scale=1e3), ATTN_EINVAL),
    ((0.03, 0.03), dict(q=None), ATTN_EINVAL), ((0.03, 0.03), dict(page=8), ATTN_EUNSUPPORTED),
    ((0.03, 0.03), dict(d=96), ATTN_EUNSUPPORTED), ((0.03, 0.03), dict(ws_bytes=WS - 1), ATTN_EINVAL),
    ((0.03, 0.03), dict(v=3 * P + 8), ATTN_EINVAL), ((0.03, 0.03), dict(Hq=34, Hkv=2), ATTN_EUNSUPPORTED),
    ((0.03, 0.03), dict(ws=2 * P), ATTN_EINVAL),             # workspace over the key pool
    ((0.03, 0.03), dict(o=P), ATTN_EINVAL),                  # output aliases q
])
def test_decode_int8_rejects_bad_arguments(scales, bad, code):
    assert _dec_i8(*scales, **bad) == code
    assert tea.attn_last_error().startswith("attn_decode_paged_int8")
