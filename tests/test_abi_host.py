"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
any device work (no GPU needed: create/bind/size functions never touch the
device, and the hot calls validate first)."""
import os
import re

import pytest

import hybrid_attention_ssm_swa_amd as H
from hybrid_attention_ssm_swa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in ("hymba_mixer.h", "griffin_block.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="library not built")

FAKE = 1 << 20   # an aligned, never-dereferenced stand-in for device pointers


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:hymba|griffin)_[a-z_]+)\s*\(", text))
    return sorted(names)


def _cfg(**kw):
    base = dict(d_model=64, n_heads=4, n_kv_heads=2, head_dim=32, d_inner=64, d_state=8, n_meta=4,
                window=8, own_kv=1, dtype=L.HYMBA_F32, rms_eps=1e-6, rope_base=0.0)
    base.update(kw)
    c = L.hymba_layer_cfg()
    for k, v in base.items():
        setattr(c, k, v)
    return c


def _weights():
    w = L.hymba_layer_weights()
    for f, _ in w._fields_:
        setattr(w, f, FAKE)
    return w


def _create(cfg):
    n = L.hymba_layer_persistent_bytes(cfg)
    assert n > 0
    return L.hymba_layer_create(cfg, _weights(), FAKE, n)


def test_every_declared_function_is_exported():
    lib = L.load_library()
    declared = _declared_functions()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(L.EXPORTED)


def test_status_strings():
    assert H.hymba_status_string(0) == "HYMBA_OK"
    assert H.hymba_status_string(-4) == "HYMBA_ERR_BIND"
    assert H.hymba_status_string(-99) == "HYMBA_UNKNOWN_STATUS"


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=3), L.HYMBA_ERR_INVALID_ARG),
    (dict(d_model=0), L.HYMBA_ERR_INVALID_ARG),
    (dict(dtype=7), L.HYMBA_ERR_INVALID_ARG),
    (dict(d_state=12), L.HYMBA_ERR_UNSUPPORTED),
    (dict(head_dim=48), L.HYMBA_ERR_UNSUPPORTED),
    (dict(dtype=L.HYMBA_BF16, head_dim=32), L.HYMBA_ERR_UNSUPPORTED),
    (dict(dtype=L.HYMBA_BF16, head_dim=64, n_heads=18, n_kv_heads=2), L.HYMBA_ERR_UNSUPPORTED),
    (dict(d_inner=60), L.HYMBA_ERR_UNSUPPORTED),
    (dict(rope_base=-1.0), L.HYMBA_ERR_INVALID_ARG),
    (dict(rope_base=float("inf")), L.HYMBA_ERR_INVALID_ARG),
])
def test_create_rejects_bad_configs(kw, code):
    cfg = _cfg(**kw)
    assert L.hymba_layer_persistent_bytes(cfg) == 0
    with pytest.raises(L.HymbaError) as e:
        L.hymba_layer_create(cfg, _weights(), FAKE, 1 << 30)
    assert e.value.status == code


def test_long_meta_prefix_is_accepted():
    assert L.hymba_layer_persistent_bytes(_cfg(dtype=L.HYMBA_BF16, head_dim=64, n_meta=200)) > 0


def test_create_checks_buffers():
    cfg = _cfg()
    n = L.hymba_layer_persistent_bytes(cfg)
    with pytest.raises(L.HymbaError) as e:
        L.hymba_layer_create(cfg, _weights(), FAKE, n - 1)
    assert e.value.status == L.HYMBA_ERR_WORKSPACE
    with pytest.raises(L.HymbaError) as e:
        L.hymba_layer_create(cfg, _weights(), FAKE + 16, n)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    w = _weights()
    w.w_o = None
    with pytest.raises(L.HymbaError) as e:
        L.hymba_layer_create(cfg, w, FAKE, n)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG


def test_layer_calls_check_alignment():
    """The kernels move rows in 16-byte vectors and carve the workspace into 256-byte regions:
    misaligned pointers are rejected before any device work."""
    cfg = _cfg()
    n = L.hymba_layer_persistent_bytes(cfg)
    w = _weights()
    w.w_in = FAKE + 2
    with pytest.raises(L.HymbaError) as e:
        L.hymba_layer_create(cfg, w, FAKE, n)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    h = _create(_cfg())
    try:
        ws = L.hymba_mixer_workspace_bytes(h, 1, 4)
        for x, y, st, wsp in [(FAKE + 8, FAKE, None, FAKE), (FAKE, FAKE + 4, None, FAKE),
                              (FAKE, FAKE, FAKE + 4, FAKE), (FAKE, FAKE, None, FAKE + 16)]:
            with pytest.raises(L.HymbaError) as e:
                L.hymba_mixer_prefill(h, x, 1, 4, y, None, st, wsp, ws, None)
            assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        kv = L.hymba_kv()
        kv.k_cache, kv.v_cache, kv.cache_len = FAKE + 2, FAKE, 16
        with pytest.raises(L.HymbaError) as e:
            L.hymba_mixer_decode(h, FAKE, FAKE, 1, FAKE, kv, FAKE, FAKE, 1 << 30, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        kv.k_cache = FAKE
        for x, pos, st, wsp in [(FAKE + 2, FAKE, FAKE, FAKE), (FAKE, FAKE + 4, FAKE, FAKE),
                                (FAKE, FAKE, FAKE + 8, FAKE), (FAKE, FAKE, FAKE, FAKE + 64)]:
            with pytest.raises(L.HymbaError) as e:
                L.hymba_mixer_decode(h, x, pos, 1, FAKE, kv, st, wsp, 1 << 30, None)
            assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        with pytest.raises(L.HymbaError) as e:
            L.hymba_layer_prepare(h, None, FAKE + 16, 1 << 30, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    finally:
        L.hymba_layer_destroy(h)


def test_bind_rules():
    prod = _create(_cfg(own_kv=1))
    cons = _create(_cfg(own_kv=0))
    cons2 = _create(_cfg(own_kv=0))
    other = _create(_cfg(own_kv=0, n_meta=5))
    try:
        for bad in [(cons, cons), (prod, cons), (cons, cons2), (other, prod)]:
            with pytest.raises(L.HymbaError) as e:
                L.hymba_kv_share_bind(*bad)
            assert e.value.status == L.HYMBA_ERR_BIND
        L.hymba_kv_share_bind(cons, prod)
        with pytest.raises(L.HymbaError) as e:       # pairs only
            L.hymba_kv_share_bind(cons2, prod)
        assert e.value.status == L.HYMBA_ERR_BIND
        L.hymba_kv_share_bind(cons, None)             # unbind frees the producer
        L.hymba_kv_share_bind(cons2, prod)
        other_rope = _create(_cfg(own_kv=0, rope_base=500.0))
        with pytest.raises(L.HymbaError) as e:
            L.hymba_kv_share_bind(other_rope, prod)
        assert e.value.status == L.HYMBA_ERR_BIND
        L.hymba_layer_destroy(other_rope)
        wrong_window = _create(_cfg(own_kv=0, window=0))
        with pytest.raises(L.HymbaError) as e:
            L.hymba_kv_share_bind(wrong_window, prod)
        assert e.value.status == L.HYMBA_ERR_BIND
        L.hymba_layer_destroy(wrong_window)
    finally:
        for h in (prod, cons, cons2, other):
            L.hymba_layer_destroy(h)


def test_workspace_grows_with_tokens():
    h = _create(_cfg())
    try:
        a = L.hymba_mixer_workspace_bytes(h, 1, 16)
        b = L.hymba_mixer_workspace_bytes(h, 2, 16)
        assert 0 < a < b
        assert L.hymba_mixer_workspace_bytes(h, 0, 16) == 0
    finally:
        L.hymba_layer_destroy(h)


def test_hot_calls_validate_before_device_work():
    h = _create(_cfg())
    cons = _create(_cfg(own_kv=0))
    try:
        ws = L.hymba_mixer_workspace_bytes(h, 1, 4)
        with pytest.raises(L.HymbaError) as e:
            L.hymba_mixer_prefill(h, FAKE, 1, 0, FAKE, None, None, FAKE, ws, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        with pytest.raises(L.HymbaError) as e:
            L.hymba_mixer_prefill(h, FAKE, 1, 4, FAKE, None, None, FAKE, ws - 1, None)
        assert e.value.status == L.HYMBA_ERR_WORKSPACE
        with pytest.raises(L.HymbaError) as e:   # consumer without K/V
            L.hymba_mixer_prefill(cons, FAKE, 1, 4, FAKE, None, None, FAKE, ws, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        kv = L.hymba_kv()
        kv.k_cache = kv.v_cache = FAKE
        kv.cache_len = 4                           # window 8 needs >= 8 slots
        with pytest.raises(L.HymbaError) as e:
            L.hymba_mixer_decode(h, FAKE, FAKE, 1, FAKE, kv, FAKE, FAKE, 1 << 30, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        with pytest.raises(L.HymbaError) as e:     # no cache at all
            L.hymba_mixer_decode(h, FAKE, FAKE, 1, FAKE, None, FAKE, FAKE, 1 << 30, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        with pytest.raises(L.HymbaError) as e:     # more sequences than a launch grid dimension holds
            L.hymba_mixer_decode(h, FAKE, FAKE, 65536, FAKE, kv, FAKE, FAKE, 1 << 30, None)
        assert e.value.status == L.HYMBA_ERR_UNSUPPORTED
        with pytest.raises(L.HymbaError) as e:
            L.hymba_layer_meta_outputs(h)          # not prepared yet
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    finally:
        L.hymba_layer_destroy(h)
        L.hymba_layer_destroy(cons)


def test_kernel_entry_points_validate():
    with pytest.raises(L.HymbaError) as e:
        L.hymba_kernel_attention(L.HYMBA_BF16, FAKE, 64, FAKE, FAKE, 64, 64, FAKE, FAKE, 4, FAKE, 64, 1, 4, 4, 2,
                                 32, 8, None)
    assert e.value.status == L.HYMBA_ERR_UNSUPPORTED
    with pytest.raises(L.HymbaError) as e:
        L.hymba_kernel_selective_scan(L.HYMBA_F32, FAKE, FAKE, 8, FAKE, 8, FAKE, FAKE, FAKE, None, FAKE, 8, None,
                                      1, 4, 8, 4, FAKE, 1 << 20, None)
    assert e.value.status == L.HYMBA_ERR_UNSUPPORTED
    with pytest.raises(L.HymbaError) as e:
        L.hymba_kernel_selective_scan(L.HYMBA_BF16, FAKE, FAKE, 8, FAKE, 8, FAKE, FAKE, FAKE, None, FAKE, 8, None,
                                      1, 4, 8, 8, FAKE, 1 << 20, None)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    with pytest.raises(L.HymbaError) as e:
        L.hymba_kernel_epilogue(L.HYMBA_F32, FAKE, 12, FAKE, 12, FAKE, 12, FAKE, FAKE, FAKE, 12, 3, 12, 1e-6, None)
    assert e.value.status == L.HYMBA_ERR_UNSUPPORTED


def test_stage_names_and_profile_read_without_recording():
    names = [L.hymba_stage_name(i) for i in range(L.HYMBA_N_STAGES)]
    assert names == ["in_proj", "kv_write", "attention", "w_o", "ssm", "epilogue", "out_proj", "convert", "rope"]
    assert L.hymba_stage_name(L.HYMBA_N_STAGES) == "unknown"
    h = _create(_cfg())
    try:
        assert L.hymba_layer_profile_read(h) == [0.0] * L.HYMBA_N_STAGES   # nothing recorded: no device call
        L.hymba_layer_profile(h, False)
    finally:
        L.hymba_layer_destroy(h)


def test_scan_entry_checks_strides():
    for ld, ld_bc, ldy, bc in [(4, 16, 8, FAKE), (8, 12, 8, FAKE), (8, 18, 8, FAKE), (8, 16, 4, FAKE),
                               (8, 16, 8, FAKE + 8)]:
        with pytest.raises(L.HymbaError) as e:
            L.hymba_kernel_selective_scan(L.HYMBA_F16, FAKE, FAKE, ld, bc, ld_bc, FAKE, FAKE, FAKE, None, FAKE, ldy,
                                          None, 1, 4, 8, 8, FAKE, 1 << 20, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG


def test_attention_entry_checks_strides():
    ok = dict(ld_q=640, ld_kv=128, stride=128 * 40, q=FAKE, o=FAKE)
    for bad in [dict(ld_q=636), dict(ld_kv=120), dict(ld_kv=130), dict(stride=128 * 40 + 4), dict(q=FAKE + 8),
                dict(o=FAKE + 2)]:
        a = dict(ok, **bad)
        with pytest.raises(L.HymbaError) as e:
            L.hymba_kernel_attention(L.HYMBA_F16, a["q"], a["ld_q"], FAKE, FAKE, a["ld_kv"], a["stride"], FAKE, FAKE,
                                     4, a["o"], 640, 1, 40, 10, 2, 64, 16, None)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG, bad


# --- the Griffin block's entry points -------------------------------------------------

def _gcfg(**kw):
    base = dict(d_model=64, d_rnn=96, dtype=L.HYMBA_F32, c=8.0)
    base.update(kw)
    c = L.griffin_block_cfg()
    for k, v in base.items():
        setattr(c, k, v)
    return c


def _gweights():
    w = L.griffin_block_weights()
    for f, _ in w._fields_:
        setattr(w, f, FAKE)
    return w


def test_griffin_workspace_grows_with_the_call():
    c = _gcfg()
    a, b = L.griffin_workspace_bytes(c, 1, 100), L.griffin_workspace_bytes(c, 4, 100)
    assert 0 < a < b and a % 256 == 0
    assert L.griffin_workspace_bytes(_gcfg(dtype=L.HYMBA_BF16), 1, 100) > 64 << 20   # + GEMM workspace
    assert L.griffin_workspace_bytes(c, 0, 5) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=0), L.HYMBA_ERR_INVALID_ARG),
    (dict(dtype=5), L.HYMBA_ERR_INVALID_ARG),
    (dict(c=0.0), L.HYMBA_ERR_INVALID_ARG),
    (dict(c=float("nan")), L.HYMBA_ERR_INVALID_ARG),
    (dict(d_rnn=100), L.HYMBA_ERR_UNSUPPORTED),
])
def test_griffin_rejects_bad_configs(kw, code):
    c = _gcfg(**kw)
    assert L.griffin_workspace_bytes(c, 1, 8) == 0
    with pytest.raises(L.HymbaError) as e:
        L.griffin_block_prefill(c, _gweights(), FAKE, FAKE, 1, 8, FAKE, None, None, None, None, FAKE, 1 << 40, None)
    assert e.value.status == code


def test_griffin_call_checks():
    c, w = _gcfg(), _gweights()
    big = 1 << 40
    # empty calls return before touching anything
    L.griffin_block_prefill(c, w, None, None, 0, 8, None, None, None, None, None, None, 0, None)
    cases = [
        (dict(ws_bytes=16), L.HYMBA_ERR_WORKSPACE),
        (dict(ws=FAKE + 16), L.HYMBA_ERR_INVALID_ARG),
        (dict(x=FAKE + 2), L.HYMBA_ERR_INVALID_ARG),
        (dict(y=None), L.HYMBA_ERR_INVALID_ARG),
        (dict(state=FAKE, state_out=FAKE), L.HYMBA_ERR_INVALID_ARG),   # aliasing needs seq == 1
        (dict(B=70000), L.HYMBA_ERR_UNSUPPORTED),
        (dict(B=1, T=3_000_000), L.HYMBA_ERR_UNSUPPORTED),    # 3e6 x 192 x 4 B > 2 GiB per sequence
    ]
    cases_bf16 = [(dict(pers=None), L.HYMBA_ERR_INVALID_ARG), (dict(pers=FAKE + 128), L.HYMBA_ERR_INVALID_ARG)]
    for kw, code in cases:
        a = dict(x=FAKE, y=FAKE, ws=FAKE, ws_bytes=big, state=None, state_out=None, B=2, T=8, pers=None)
        a.update(kw)
        with pytest.raises(L.HymbaError) as e:
            L.griffin_block_prefill(c, w, a["pers"], a["x"], a["B"], a["T"], a["y"], a["state"], None, a["state_out"],
                                    None, a["ws"], a["ws_bytes"], None)
        assert e.value.status == code, (kw, L.hymba_last_error())
    nw = _gweights()
    nw.lam = None
    with pytest.raises(L.HymbaError) as e:
        L.griffin_block_prefill(c, nw, None, FAKE, 1, 8, FAKE, None, None, None, None, FAKE, big, None)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    with pytest.raises(L.HymbaError) as e:
        L.griffin_block_decode(c, w, None, FAKE, 1, FAKE, None, FAKE, FAKE, big, None)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG
    cb = _gcfg(dtype=L.HYMBA_BF16)
    for kw, code in cases_bf16:
        with pytest.raises(L.HymbaError) as e:
            L.griffin_block_prefill(cb, w, kw["pers"], FAKE, 1, 8, FAKE, None, None, None, None, FAKE, big, None)
        assert e.value.status == code


def test_griffin_persistent_buffer():
    assert L.griffin_block_persistent_bytes(_gcfg()) == 0
    c = _gcfg(dtype=L.HYMBA_BF16)
    n = L.griffin_block_persistent_bytes(c)
    assert n >= 2 * (2 * 96 * 64 + 2 * 96 * 96 + 64 * 96) and n % 256 == 0
    L.griffin_block_prepare(_gcfg(), _gweights(), None, 0, None)    # fp32: nothing to do
    with pytest.raises(L.HymbaError) as e:
        L.griffin_block_prepare(c, _gweights(), FAKE, n - 1, None)
    assert e.value.status == L.HYMBA_ERR_WORKSPACE
    with pytest.raises(L.HymbaError) as e:
        L.griffin_block_prepare(c, _gweights(), FAKE + 16, n, None)
    assert e.value.status == L.HYMBA_ERR_INVALID_ARG


def test_gemm_rows_rejects_bad_arguments():
    """Validated before any device work (fake aligned pointers)."""
    args = dict(w=FAKE, ldw=8, x=FAKE, ldx=8, y=FAKE, ldy=8, y32=None, ldy32=0, c0=0, c1=0, M=1, N=8, K=8,
                ws=None, ws_bytes=0)
    cases = [
        (dict(types=(L.HYMBA_F32, L.HYMBA_F16, L.HYMBA_F16)), L.HYMBA_ERR_UNSUPPORTED),
        (dict(N=6), L.HYMBA_ERR_UNSUPPORTED),
        (dict(K=12, ldw=16, ldx=16), L.HYMBA_ERR_UNSUPPORTED),
        (dict(ldx=4), L.HYMBA_ERR_INVALID_ARG),
        (dict(x=FAKE + 8), L.HYMBA_ERR_INVALID_ARG),
        (dict(y32=FAKE, ldy32=4, c0=0, c1=8), L.HYMBA_ERR_INVALID_ARG),   # ldy32 < c1 - c0
        (dict(y=None), L.HYMBA_ERR_INVALID_ARG),
    ]
    for kw, code in cases:
        a = dict(args, types=(L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_F16))
        a.update(kw)
        with pytest.raises(L.HymbaError) as e:
            L.hymba_kernel_gemm_rows(*a["types"], a["w"], a["ldw"], a["x"], a["ldx"], a["y"], a["ldy"], a["y32"],
                                     a["ldy32"], a["c0"], a["c1"], a["M"], a["N"], a["K"], a["ws"], a["ws_bytes"],
                                     None)
        assert e.value.status == code, (kw, L.hymba_last_error())
    # zero rows: nothing to do
    L.hymba_kernel_gemm_rows(L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_F16, FAKE, 8, FAKE, 8, FAKE, 8, None, 0, 0, 0,
                             0, 8, 8, None, 0, None)
    # K is never split across workgroups: no workspace at any shape
    assert L.hymba_kernel_gemm_rows_workspace(128, 1600, 3200) == 0
    assert L.hymba_kernel_gemm_rows_workspace(300, 1600, 3200) == 0
    assert L.hymba_kernel_gemm_rows_workspace(128, 16384, 512) == 0


def test_gemm_tiles_rejects_bad_arguments():
    """Validated before any device work (fake aligned pointers)."""
    args = dict(w=FAKE, ldw=8, x=FAKE, ldx=8, y=FAKE, ldy=8, y32=None, ldy32=0, c0=0, c1=0, M=1, N=8, K=8)
    cases = [
        (dict(types=(L.HYMBA_F32, L.HYMBA_F16)), L.HYMBA_ERR_UNSUPPORTED),
        (dict(types=(L.HYMBA_BF16, L.HYMBA_F32)), L.HYMBA_ERR_UNSUPPORTED),
        (dict(N=6), L.HYMBA_ERR_UNSUPPORTED),
        (dict(K=12, ldw=16, ldx=16), L.HYMBA_ERR_UNSUPPORTED),
        (dict(ldx=4), L.HYMBA_ERR_INVALID_ARG),
        (dict(ldy=6), L.HYMBA_ERR_INVALID_ARG),
        (dict(x=FAKE + 8), L.HYMBA_ERR_INVALID_ARG),
        (dict(y=FAKE + 4), L.HYMBA_ERR_INVALID_ARG),
        (dict(y32=FAKE, ldy32=4, c0=0, c1=8), L.HYMBA_ERR_INVALID_ARG),   # ldy32 < c1 - c0
        (dict(y32=FAKE, ldy32=8, c0=2, c1=6), L.HYMBA_ERR_INVALID_ARG),   # c0, c1 not multiples of 4
        (dict(y=None), L.HYMBA_ERR_INVALID_ARG),
        (dict(M=-1), L.HYMBA_ERR_INVALID_ARG),
    ]
    for kw, code in cases:
        a = dict(args, types=(L.HYMBA_BF16, L.HYMBA_F16))
        a.update(kw)
        with pytest.raises(L.HymbaError) as e:
            L.hymba_kernel_gemm_tiles(*a["types"], a["w"], a["ldw"], a["x"], a["ldx"], a["y"], a["ldy"], a["y32"],
                                      a["ldy32"], a["c0"], a["c1"], a["M"], a["N"], a["K"], None)
        assert e.value.status == code, (kw, L.hymba_last_error())
    # zero rows: nothing to do
    L.hymba_kernel_gemm_tiles(L.HYMBA_F16, L.HYMBA_F16, FAKE, 8, FAKE, 8, FAKE, 8, None, 0, 0, 0, 0, 8, 8, None)


def test_scan_workspace_sizes():
    """The scan's workspace: the scaled A (E*N fp32, 256-byte aligned), plus (S - 1) segment
    summaries of B*E*(N + 1) fp32 when too few channel groups would fill the GPU: S segments of a
    multiple of 16 steps, S <= 8, each >= 256 steps, enough for ~3072 waves at 4 states per wave."""
    ws = L.hymba_kernel_selective_scan_workspace
    # 1.5B 8K SWA prefill: 16 x 50 channel groups x 4 waves = 3200 waves, one pass
    assert ws(16, 8192, 3200, 16) == 3200 * 16 * 4
    # global 8K prefill, B = 8: 1600 waves -> 2 segments of 4096 steps
    assert ws(8, 8192, 3200, 16) == 3200 * 16 * 4 + 1 * 8 * 3200 * 17 * 4
    # 300M ablation, B = 8, T = 2048: 1024 waves -> 3 segments of 688 steps
    assert ws(8, 2048, 2048, 16) == 2048 * 16 * 4 + 2 * 8 * 2048 * 17 * 4
    # short sequences never split (segments of >= 256 steps)
    assert ws(1, 300, 520, 16) == 520 * 16 * 4
    assert ws(2, 511, 520, 8) == 520 * 8 * 4 + 256 * 0   # 511 // 256 = 1 segment
    assert ws(2, 1100, 520, 8) == 520 * 8 * 4 + 3 * 2 * 520 * 9 * 4   # 4 segments of 288 steps
    assert ws(1, 100000, 64, 16) == 64 * 16 * 4 + 7 * 1 * 64 * 17 * 4   # at most 8 segments
    assert ws(0, 10, 64, 16) == 0 and ws(1, 10, 64, 12) == 0


def test_check_and_overlap_calls():
    lib = L.load_library()
    assert lib.hymba_layer_check(None, None) == L.HYMBA_ERR_INVALID_ARG
    assert lib.hymba_layer_set_overlap(None, 1) == L.HYMBA_ERR_INVALID_ARG
    assert lib.hymba_layer_set_gemm(None, 0) == L.HYMBA_ERR_INVALID_ARG
    assert H.hymba_status_string(L.HYMBA_ERR_RANGE) == "HYMBA_ERR_RANGE"
    h = _create(_cfg())
    try:
        L.hymba_layer_set_overlap(h, False)     # host only
        L.hymba_layer_set_overlap(h, True)
        L.hymba_layer_set_gemm(h, L.HYMBA_GEMM_TILED)
        L.hymba_layer_set_gemm(h, L.HYMBA_GEMM_LIBRARY)
        with pytest.raises(L.HymbaError) as e:
            L.hymba_layer_set_gemm(h, 2)
        assert e.value.status == L.HYMBA_ERR_INVALID_ARG
        L.hymba_layer_check(h, None)            # nothing has run on the device: no device call, OK
    finally:
        L.hymba_layer_destroy(h)
