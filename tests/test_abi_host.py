"""The C ABI on the host: exports, sizing, validation, and the append/merge
bookkeeping of a host-only pool against the oracle's closed-form schedule.

No compute call runs here (a host-only pool enqueues nothing)."""

import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_recurrent_dl_amd as dl
from linear_attention_recurrent_dl_amd import _native as N
from oracle import schedule
from workloads import CONFIGS, Workload, small_variant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltalog.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|const char \*)\s*(dl_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = N.lib()
    names = header_functions()
    assert len(names) >= 13, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in deltalog.h but not exported"
    assert set(names) == set(N.EXPORTED)


def test_binding_names_match_c_names():
    for name in header_functions():
        assert callable(getattr(dl, name)), name


def _desc(**kw):
    base = dict(num_slots=8, max_batch=4, H_v=4, H_k=2, d=64, L=8, decay="per_key",
                update="delta", state_dtype="f32", in_dtype="bf16")
    base.update(kw)
    return dl.make_desc(**base)


def test_pool_sizes_formula():
    for cfg in CONFIGS.values():
        desc = dl.make_desc(cfg.num_slots, cfg.batch, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay,
                            cfg.update, cfg.state_dtype, cfg.in_dtype)
        sz = dl.dl_pool_sizes(desc)
        P, Hv, Hk, D, C = cfg.num_slots, cfg.H_v, cfg.H_k, cfg.d, cfg.L - 1
        s_st = 2 if cfg.state_dtype == "bf16" else 4
        s_in = 2 if cfg.in_dtype == "bf16" else 4
        s_b = 4 if cfg.update == "delta" else s_in
        lam_w = {"none": 0, "scalar": 1, "per_key": D}[cfg.decay]
        bv = dl.dl_value_tile(desc)
        units = cfg.batch * Hv
        if D <= 32 or units >= 256:
            want = D
        elif D == 128 and units < 64:
            want = 16
        elif D == 128 and cfg.state_dtype == "f32" and units >= 128:
            want = 64
        else:
            want = 32
        assert bv == want, cfg.name
        assert sz == [P * Hv * D * D * s_st, P * Hk * C * D * s_in, P * Hv * C * D * s_b,
                      P * Hv * C * lam_w * 4, P * Hv * (D // bv) * 4, 0], cfg.name
        # split replay adds one launch's coefficient scratch: 2 L floats per (entry, v-head)
        split = dl.make_desc(cfg.num_slots, cfg.batch, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay,
                             cfg.update, cfg.state_dtype, cfg.in_dtype, replay_split=1)
        launch_slots = min(cfg.batch, dl.dl_launch_slot_limit())
        assert dl.dl_pool_sizes(split) == sz[:5] + [launch_slots * Hv * 2 * cfg.L * 4], cfg.name


@pytest.mark.parametrize("d,bv,ok", [(128, 128, True), (128, 64, True), (128, 32, True), (128, 16, True),
                                     (128, 8, False), (128, 48, False), (64, 64, True), (64, 32, True),
                                     (64, 16, False), (32, 32, True), (32, 16, False), (16, 16, True)])
def test_value_tile_choices(d, bv, ok):
    desc = dl.make_desc(4, 4, 2, 2, d, 4, "scalar", "delta", "f32", "f32", value_tile=bv)
    if ok:
        assert dl.dl_value_tile(desc) == bv
        assert dl.dl_pool_sizes(desc)[4] == 4 * 2 * (d // bv) * 4
    else:
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_value_tile(desc)
        assert ei.value.code == N.DL_ERR_UNSUPPORTED


@pytest.mark.parametrize("d,state,batch,heads,want", [
    (128, "f32", 1, 32, 16), (128, "f32", 2, 32, 32), (128, "f32", 4, 32, 64), (128, "f32", 7, 32, 64),
    (128, "f32", 8, 32, 128), (128, "f32", 512, 32, 128), (128, "bf16", 1, 32, 16), (128, "bf16", 4, 32, 32),
    (128, "bf16", 256, 32, 128), (64, "f32", 1, 32, 32), (64, "f32", 8, 32, 64), (32, "f32", 1, 2, 32),
    (16, "f32", 1, 2, 16)])
def test_default_value_tile(d, state, batch, heads, want):
    """Narrow tiles while a launch's slot-heads would give fewer than 256
    blocks, whole rows beyond (per-key decay; fp32 and eager pools alike)."""
    desc = dl.make_desc(batch, batch, heads, heads, d, 16, "per_key", "delta", state, "f32")
    assert dl.dl_value_tile(desc) == want
    assert dl.dl_value_tile(dl.make_desc(batch, batch, heads, heads, d, 1, "scalar", "delta", state,
                                         "bf16")) == want


@pytest.mark.parametrize("batch,want", [(1, 16), (4, 32), (8, 64), (32, 64), (63, 64), (64, 128), (256, 128)])
def test_default_value_tile_bf16_state_with_log(batch, want):
    """A bf16 state with a log and a scalar decay keeps 64-column tiles up to
    2047 slot-heads (32 v-heads here); an eager pool (L = 1) of the same shape
    takes whole rows from 256 slot-heads."""
    desc = dl.make_desc(batch, batch, 32, 16, 128, 16, "scalar", "delta", "bf16", "bf16")
    assert dl.dl_value_tile(desc) == want
    eager = dl.make_desc(batch, batch, 32, 16, 128, 1, "scalar", "delta", "bf16", "bf16")
    assert dl.dl_value_tile(eager) == (want if batch * 32 < 256 else 128)


@pytest.mark.parametrize("field,value,code", [
    ("num_slots", 0, N.DL_ERR_INVALID_ARG),
    ("num_slots", (1 << 24) + 1, N.DL_ERR_INVALID_ARG),   # slot ids travel in 24 bits
    ("max_batch", 0, N.DL_ERR_INVALID_ARG),
    ("num_v_heads", 3, N.DL_ERR_INVALID_ARG),       # not a multiple of H_k = 2
    ("num_v_heads", 32770, N.DL_ERR_INVALID_ARG),   # q/k head index exact up to 2^15 v-heads
    ("num_slots", 1 << 24, N.DL_ERR_INVALID_ARG),     # with 128 v-heads: 2^31 (slot-head, tile) units
    ("num_k_heads", 0, N.DL_ERR_INVALID_ARG),
    ("merge_interval", 0, N.DL_ERR_INVALID_ARG),
    ("merge_interval", 65, N.DL_ERR_INVALID_ARG),
    ("decay", 7, N.DL_ERR_INVALID_ARG),
    ("update", 2, N.DL_ERR_INVALID_ARG),
    ("state_dtype", 5, N.DL_ERR_INVALID_ARG),
    ("replay_split", 2, N.DL_ERR_INVALID_ARG),
    ("d_k", 48, N.DL_ERR_UNSUPPORTED),
    ("d_v", 32, N.DL_ERR_UNSUPPORTED),                # d_k != d_v
])
def test_descriptor_validation(field, value, code):
    desc = _desc()
    setattr(desc, field, value)
    if field == "d_k":
        desc.d_v = value
    if field == "num_slots" and value == 1 << 24:
        desc.num_v_heads = 128
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_pool_sizes(desc)
    assert ei.value.code == code
    with pytest.raises(dl.DeltaLogError):
        dl.dl_pool_create(desc, None)


def test_create_rejects_missing_or_misaligned_buffers():
    desc = _desc()
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_pool_create(desc, N.dl_pool_buffers(None, None, None, None, None))
    assert ei.value.code == N.DL_ERR_INVALID_ARG
    with pytest.raises(dl.DeltaLogError):
        dl.dl_pool_create(desc, N.dl_pool_buffers(16, 32, 48, 64, 72))   # 72 not 16-aligned


def _host_pool(**kw):
    d = dict(num_slots=8, H_v=4, H_k=2, d=64, L=8, decay="per_key", update="delta",
             state_dtype="f32", in_dtype="bf16", max_batch=4, device=None)
    d.update(kw)
    return dl.DeltaLogPool(**d)


def test_errors_leave_pool_unchanged():
    p = _host_pool()
    p.decode_step([0, 1, 2])
    before = p.log_len().copy()
    cases = [([1, 1], N.DL_ERR_DUPLICATE_SLOT), ([0, 8], N.DL_ERR_SLOT_RANGE),
             ([-1], N.DL_ERR_SLOT_RANGE), ([0, 1, 2, 3, 4], N.DL_ERR_BATCH_TOO_LARGE)]
    for ids, code in cases:
        for call in (p.decode_step, p.merge, p.assign):
            with pytest.raises(dl.DeltaLogError) as ei:
                call(ids)
            assert ei.value.code == code, (ids, call)
            assert np.array_equal(p.log_len(), before)
    with pytest.raises(dl.DeltaLogError) as ei:
        p.schedule([3, 3])
    assert ei.value.code == N.DL_ERR_DUPLICATE_SLOT


def test_token_pointer_rules():
    lib = N.lib()
    ids = np.array([0], dtype=np.int32)
    ip = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p_none = _host_pool(decay="none", update="plain")
    # lambda must be NULL without decay; beta NULL for plain
    assert lib.dl_decode_step(p_none.handle, 1, ip, None, None, None, 16, None, None, None) == N.DL_ERR_INVALID_ARG
    assert lib.dl_decode_step(p_none.handle, 1, ip, None, None, None, None, 16, None, None) == N.DL_ERR_INVALID_ARG
    assert p_none.log_len().tolist() == [0] * 8
    # eager step needs L == 1
    p = _host_pool()
    with pytest.raises(dl.DeltaLogError):
        p.eager_step([0])
    pe = _host_pool(L=1)
    pe.eager_step([0, 1])
    assert pe.log_len().tolist() == [0] * 8
    # zero-length calls are no-ops
    p.decode_step([])
    p.merge([])
    p.assign([])
    assert p.log_len().tolist() == [0] * 8
    with pytest.raises(dl.DeltaLogError) as ei:
        p.device_log_len()
    assert ei.value.code == N.DL_ERR_DRY_RUN


def test_read_base_rules():
    lib = N.lib()
    p = _host_pool()
    ids = np.array([0, 1], dtype=np.int32)
    ip = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    # a host-only pool has no device state to read
    assert lib.dl_read_base(p.handle, 2, ip, 16, None) == N.DL_ERR_DRY_RUN
    # slot validation comes first, as for every slot call
    dup = np.array([1, 1], dtype=np.int32)
    assert lib.dl_read_base(p.handle, 2, dup.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 16,
                            None) == N.DL_ERR_DUPLICATE_SLOT
    big = np.arange(5, dtype=np.int32)
    assert lib.dl_read_base(p.handle, 5, big.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 16,
                            None) == N.DL_ERR_BATCH_TOO_LARGE
    assert lib.dl_read_base(None, 2, ip, 16, None) == N.DL_ERR_INVALID_ARG
    assert p.log_len().tolist() == [0] * 8


@pytest.mark.parametrize("L", [1, 2, 5, 16])
def test_host_schedule_matches_closed_form(L):
    rng = np.random.default_rng(L)
    P = 12
    p = _host_pool(num_slots=P, L=L, max_batch=P)
    cnt = schedule.Counters(P, L)
    for t in range(80):
        if t % 9 == 4:
            rs = rng.choice(P, size=3, replace=False)
            p.assign(rs)
            cnt.reset(rs)
        if t % 13 == 6:
            ms = rng.choice(P, size=4, replace=False)
            p.merge(ms)
            cnt.merge(ms)
        if t % 29 == 28:
            p.flush_all()
            cnt.merge(np.arange(P))
        B = int(rng.integers(0, P + 1))
        ids = rng.choice(P, size=B, replace=False)
        merge, index = p.schedule(ids)
        want = cnt.decode(ids)
        assert merge.tolist() == [int(ph == schedule.MERGE) for ph, _ in want]
        assert index.tolist() == [ix for _, ix in want]
        p.decode_step(ids)
        assert np.array_equal(p.log_len(), cnt.n)


def test_host_schedule_serving_pool_workload():
    """The serving-pool workload's bookkeeping (ragged fill, 51 replacements and
    256 random slots per step) on a host-only pool, step by step."""
    cfg = small_variant(CONFIGS[5], steps=64)
    wl = Workload(cfg)
    p = dl.DeltaLogPool(cfg.num_slots, cfg.H_v, cfg.H_k, cfg.d, cfg.L, cfg.decay, cfg.update,
                        cfg.state_dtype, cfg.in_dtype, max_batch=cfg.batch, device=None)
    cnt = schedule.Counters(cfg.num_slots, cfg.L)
    for desc in wl.plan():
        inp = wl.step_inputs(desc)
        if len(inp.replace_ids):
            p.assign(inp.replace_ids)
            cnt.reset(inp.replace_ids)
        merge, index = p.schedule(inp.slot_ids)
        want = cnt.decode(inp.slot_ids)
        assert merge.tolist() == [int(ph == schedule.MERGE) for ph, _ in want]
        assert index.tolist() == [ix for _, ix in want]
        p.decode_step(inp.slot_ids)
        assert np.array_equal(p.log_len(), cnt.n)
    # after the fill phase every slot had its drawn initial fill
    wl2 = Workload(cfg)
    cnt2 = schedule.Counters(cfg.num_slots, cfg.L)
    for desc in wl2.fill_steps():
        cnt2.decode(desc.slots)
    assert np.array_equal(cnt2.n, wl2.initial_fill())


def test_merge_sweep_shapes_validate():
    """Every merge-sweep shape is accepted.  At M = 64 the live log of a
    whole-row tile exceeds the 56 KiB LDS budget, and the default falls back to
    the widest tile that fits.  KDA's 63 entries (bf16 keys, fp32 values and
    per-key snapshots) need 80,640 B at 128 columns and 64,512 B at 64, so it
    gets 32 columns (56,448 B); an explicit wider tile is refused up front."""
    from workloads import SWEEP_OPERATORS, merge_sweep_config
    for op in SWEEP_OPERATORS:
        for M in (1, 2, 4, 8, 16, 32, 64):
            c = merge_sweep_config(op, M)
            desc = dl.make_desc(c.num_slots, c.batch, c.H_v, c.H_k, c.d, M, c.decay, c.update,
                                c.state_dtype, c.in_dtype)
            assert dl.dl_pool_sizes(desc)[0] == c.num_slots * c.H_v * c.d * c.d * 4
            s_in = 2 if c.in_dtype == "bf16" else 4
            s_b = 4 if c.update == "delta" else s_in
            snap = c.d * 4 if c.decay == "per_key" else 0
            want = next(bv for bv in (128, 64, 32, 16)
                        if (M - 1) * (c.d * s_in + bv * s_b + snap) <= 56 * 1024 or bv == 16)
            assert dl.dl_value_tile(desc) == want, (op, M)
            assert want == 128 or M == 64
            if M == 64 and op == "kda":
                for bv in (128, 64):
                    wide = dl.make_desc(c.num_slots, c.batch, c.H_v, c.H_k, c.d, M, c.decay, c.update,
                                        c.state_dtype, c.in_dtype, value_tile=bv)
                    with pytest.raises(dl.DeltaLogError) as ei:
                        dl.dl_pool_sizes(wide)
                    assert ei.value.code == N.DL_ERR_UNSUPPORTED


def test_decode_window_rules():
    """dl_decode_window on a host-only pool: argument checks before anything
    changes, then every windowed slot's log is empty and the others keep theirs."""
    lib = N.lib()
    p = _host_pool()                                     # per-key decay, delta, L = 8
    ids = np.array([0, 1, 2], dtype=np.int32)
    ip = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    for _ in range(3):
        p.decode_step([0, 1, 2, 3])
    before = p.log_len().tolist()
    assert before == [3, 3, 3, 3, 0, 0, 0, 0]
    for W in (0, -1, 4097):
        assert lib.dl_decode_window(p.handle, 3, ip, W, None, None, None, None, None, None, None) \
            == N.DL_ERR_INVALID_ARG
    dup = np.array([1, 1], dtype=np.int32)
    assert lib.dl_decode_window(p.handle, 2, dup.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 4, None, None,
                                None, None, None, None, None) == N.DL_ERR_DUPLICATE_SLOT
    big = np.arange(5, dtype=np.int32)
    assert lib.dl_decode_window(p.handle, 5, big.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 4, None, None,
                                None, None, None, None, None) == N.DL_ERR_BATCH_TOO_LARGE
    assert p.log_len().tolist() == before                # refused calls change nothing
    p.decode_window([0, 2], 5)
    assert p.log_len().tolist() == [0, 3, 0, 3, 0, 0, 0, 0]
    # the schedule continues from an empty log
    p.decode_step([0, 1])
    assert p.log_len().tolist() == [1, 4, 0, 3, 0, 0, 0, 0]
    # lambda / beta presence follows the operator, as for a step
    q = _host_pool(decay="none", update="plain")
    one = np.array([0], dtype=np.int32)
    op = one.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.dl_decode_window(q.handle, 1, op, 2, None, None, None, 16, None, None, None) == N.DL_ERR_INVALID_ARG
    assert lib.dl_decode_window(q.handle, 1, op, 2, None, None, None, None, 16, None, None) == N.DL_ERR_INVALID_ARG
    assert lib.dl_decode_window(q.handle, 0, op, 2, None, None, None, None, None, None, None) == N.DL_OK


def test_qk_head_multiplier_is_exact_up_to_the_head_limit():
    """The kernels find the q/k head of v-head h as the high word of
    2h * ceil(2^31 / G), G = H_v / H_k, and the group's first v-head as the
    one whose q/k head differs from that of h - 1 (unsigned, so h = 0 wraps).
    Checked over every h for group sizes up to the pool's 32768 v-heads."""
    import numpy as np
    limit = 32768
    for G in sorted({1, 2, 3, 5, 7, 8, 16, 31, 127, 1000, 4095, 4096, 16383, 32767, 32768}):
        H_v = (limit // G) * G
        m = (2 ** 31 + G - 1) // G
        h = np.arange(H_v, dtype=np.uint64)
        g = ((2 * h) * m) >> np.uint64(32)
        assert np.array_equal(g, h // G), G
        prev = (((2 * h - 2) % 2 ** 32) * m) >> np.uint64(32)
        assert np.array_equal(g != prev, h % G == 0), G
