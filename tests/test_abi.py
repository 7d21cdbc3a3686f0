"""Host-side tests of the C ABI: the library loads and exports every declared
symbol, size arithmetic, workspace queries, and argument validation (every
rejected call returns before any launch, so these run without a GPU)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest
import torch

import mla_latent_kv_12_amd as mla
from mla_latent_kv_12_amd import binding, datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "cache_tables.json")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_struct_layouts_match_header():
    # field order and C sizes: int64 x 11, float, int32 x 3, double
    assert ctypes.sizeof(binding.DecodeParams) == 11 * 8 + 4 * 4 + 8
    assert binding.DecodeParams.q_rope_base.offset == 104
    assert ctypes.sizeof(binding.PrefillParams) == 12 * 8 + 4 * 4 + 8
    assert binding.PrefillParams.q_rope_base.offset == 112
    assert ctypes.sizeof(binding.AppendParams) == 9 * 8 + 8 + 2 * 4   # + double rope_base


def test_kv_cache_bytes_reproduces_the_pages():
    g = json.load(open(GOLDEN))
    for row in g["eyestech_telemetry"]["rows"]:
        w = row["elems_per_token"]
        for s, gib in zip(g["eyestech_telemetry"]["seq_lens"], row["gib"]):
            assert round(mla.kv_cache_bytes(60, 8, s, row.get("d_c", w), row.get("d_r", 0), 2)
                         / 2**30, 2) == gib
    assert mla.kv_cache_bytes(1, 1, 1, 512, 64, 1) == 576
    assert mla.kv_cache_bytes(60, 1, 131072, 512, 64, 2) / 2**30 == pytest.approx(8.4375)
    assert mla.kv_cache_bytes(-1, 1, 1, 1, 1, 1) == 0


def test_status_strings_and_version():
    for s in range(5):
        assert mla.status_string(s).startswith("MLA_")
    assert mla.version() >= 10000


def _v3_params(**kw):
    base = dict(batch=8, heads=128, d_c=512, d_r=64, d_n=128, d_v=128, n_max=131072,
                ckv_stride_b=131072 * 576, ckv_stride_n=576, kpe_stride_b=131072 * 576,
                kpe_stride_n=576, softmax_scale=0.0, dtype=mla.MLA_BF16, out_dtype=mla.MLA_BF16,
                num_splits=0)
    base.update(kw)
    return binding.DecodeParams(**base)


def test_decode_workspace_size():
    p = _v3_params(num_splits=32)
    ws = mla.decode_workspace_bytes(p)
    q = 8 * 128 * 576 * 2
    o = 8 * 32 * 128 * 512 * 4
    ml = 8 * 32 * 128 * 2 * 4
    lat = 8 * 128 * 512 * 4        # merged latents for the batched up-projection (B*H >= 1024)
    plan = lambda items, rows: rnd(items * 16) + rnd(rows * 8)   # item and row tables
    rnd = lambda x: (x + 255) // 256 * 256
    assert ws == rnd(q) + rnd(o) + rnd(ml) + rnd(lat) + plan(8 * 32, 8)
    # batch 4 (B*H = 512) keeps the fused merge + up-projection: no latent buffer
    assert mla.decode_workspace_bytes(_v3_params(batch=4, num_splits=32)) == \
        rnd(q // 2) + rnd(o // 2) + rnd(ml // 2) + plan(4 * 32, 4)
    # the balanced plan (num_splits = 0) sizes its partials for 256 items
    # (one per compute unit) whatever the batch below 256
    for batch in (1, 8, 100):
        got = mla.decode_workspace_bytes(_v3_params(batch=batch))
        qb = batch * 128 * 576 * 2
        latb = batch * 128 * 512 * 4 if batch * 128 >= 1024 else 0
        assert got == rnd(qb) + rnd(256 * 128 * 512 * 4) + rnd(256 * 128 * 8) + rnd(latb) + \
            plan(256, batch)
    # 300 sequences: one item each at most
    assert mla.decode_workspace_bytes(_v3_params(batch=300)) == \
        rnd(300 * 128 * 576 * 2) + rnd(300 * 128 * 512 * 4) + rnd(300 * 128 * 8) + \
        rnd(300 * 128 * 512 * 4) + plan(300, 300)
    # the bf16 path rotates q_rope while placing it beside q~ (no extra room);
    # the fp32 path keeps a rotated copy
    assert mla.decode_workspace_bytes(_v3_params(num_splits=32, q_rope_base=10000.0)) == ws
    f32 = dict(dtype=mla.MLA_F32, out_dtype=mla.MLA_F32, num_splits=32)
    assert mla.decode_workspace_bytes(_v3_params(q_rope_base=10000.0, **f32)) == \
        mla.decode_workspace_bytes(_v3_params(**f32)) + rnd(8 * 128 * 64 * 4)
    # the fp32 path has no plan tables
    assert mla.decode_workspace_bytes(_v3_params(**f32)) == \
        rnd(8 * 128 * 512 * 4) + rnd(8 * 32 * 128 * 512 * 4) + rnd(8 * 32 * 128 * 8)
    assert mla.decode_workspace_bytes(_v3_params()) > 0            # auto split count
    assert mla.decode_workspace_bytes(_v3_params(d_c=256)) == 0    # unsupported -> 0
    assert mla.decode_workspace_bytes(_v3_params(batch=0)) == 0


def _call_decode(p, ptrs=None, ws_bytes=1 << 40, ws=0x100000):
    lib = binding.lib()
    fake = ptrs or dict(q_nope=0x1000, q_rope=0x2000, w_uk=0x3000, w_uv=0x4000, ckv=0x5000,
                        kpe=0x5400, seqlens=0x6000, out=0x7000)
    vp = ctypes.c_void_p
    return lib.mla_decode(ctypes.byref(p), vp(fake["q_nope"]), vp(fake["q_rope"]),
                          vp(fake["w_uk"]), vp(fake["w_uv"]), vp(fake["ckv"]), vp(fake["kpe"]),
                          vp(fake["seqlens"]), vp(fake["out"]), vp(ws), ws_bytes, None)


def _msg():
    return binding.lib().mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), mla.MLA_ERR_INVALID_ARG),
    (dict(heads=0), mla.MLA_ERR_INVALID_ARG),
    (dict(d_r=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(d_c=256), mla.MLA_ERR_UNSUPPORTED),
    (dict(heads=96), mla.MLA_ERR_UNSUPPORTED),
    (dict(d_n=64), mla.MLA_ERR_UNSUPPORTED),
    (dict(dtype=7), mla.MLA_ERR_UNSUPPORTED),
    (dict(out_dtype=3), mla.MLA_ERR_UNSUPPORTED),
    (dict(ckv_stride_n=500), mla.MLA_ERR_INVALID_ARG),
    (dict(ckv_stride_b=576), mla.MLA_ERR_INVALID_ARG),
    (dict(num_splits=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(num_splits=100000), mla.MLA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(q_rope_base=1.0), mla.MLA_ERR_INVALID_ARG),
    (dict(q_rope_base=-2.0), mla.MLA_ERR_INVALID_ARG),
    (dict(q_rope_base=float("inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(ckv_stride_n=580, kpe_stride_n=580, ckv_stride_b=131072 * 580,
          kpe_stride_b=131072 * 580), mla.MLA_ERR_INVALID_ARG),  # rows not 16-byte aligned
    # strides whose products with n_max or the batch would overflow 64 bits
    (dict(ckv_stride_n=1 << 55), mla.MLA_ERR_UNSUPPORTED),
    (dict(kpe_stride_b=1 << 62), mla.MLA_ERR_UNSUPPORTED),
    (dict(ckv_stride_b=-576), mla.MLA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_params_before_launch(kw, status):
    assert _call_decode(_v3_params(**kw)) == status
    assert _msg() != ""


def test_decode_rejects_null_and_misaligned_pointers():
    p = _v3_params()
    ptrs = dict(q_nope=0x1000, q_rope=0x2000, w_uk=0x3000, w_uv=0x4000, ckv=0x5000, kpe=0x5400,
                seqlens=0x6000, out=0x7000)
    for k in ("q_nope", "w_uk", "w_uv", "ckv", "seqlens", "out", "q_rope", "kpe"):
        bad = dict(ptrs, **{k: 0})
        assert _call_decode(p, bad) == mla.MLA_ERR_INVALID_ARG, k
    assert _call_decode(p, dict(ptrs, ckv=0x5002)) == mla.MLA_ERR_INVALID_ARG
    assert "aligned" in _msg()


def test_decode_rejects_bad_workspace():
    p = _v3_params(num_splits=8)
    need = mla.decode_workspace_bytes(p)
    assert _call_decode(p, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE
    assert _call_decode(p, ws=0) == mla.MLA_ERR_WORKSPACE
    assert _call_decode(p, ws=0x100010) == mla.MLA_ERR_WORKSPACE   # not 256-byte aligned
    assert str(need) in _msg()


def test_noalloc_decode_refuses_before_any_launch():
    """mla_decode_noalloc checks its arguments and the size of its fixed
    scratch on the host first: a call that would need more than
    MLA_DECODE_NOALLOC_MAX_BYTES, or with bad arguments, returns before any
    device call (so this runs without a GPU)."""
    lib = binding.lib()
    vp = ctypes.c_void_p
    ptrs = [vp(x) for x in (0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x5400, 0x6000, 0x7000)]

    def call(p, args=ptrs):
        return lib.mla_decode_noalloc(ctypes.byref(p), *args, None)

    # the V3 128k decode at batch 8 fits with the library's split count; 64 splits do not
    assert mla.decode_workspace_bytes(_v3_params()) <= mla.NOALLOC_MAX_BYTES
    big = _v3_params(num_splits=64)
    need = mla.decode_workspace_bytes(big)
    assert need > mla.NOALLOC_MAX_BYTES
    assert call(big) == mla.MLA_ERR_WORKSPACE
    assert str(need) in _msg() and str(mla.NOALLOC_MAX_BYTES) in _msg()
    assert call(_v3_params(num_splits=-1)) == mla.MLA_ERR_INVALID_ARG
    assert call(_v3_params(d_c=256)) == mla.MLA_ERR_UNSUPPORTED
    assert call(_v3_params(), [vp(0)] + ptrs[1:]) == mla.MLA_ERR_INVALID_ARG
    header = open(HEADER).read()
    assert re.search(r"#define MLA_DECODE_NOALLOC_MAX_BYTES \(\(size_t\)80 << 20\)", header)
    assert mla.NOALLOC_MAX_BYTES == 80 << 20


def test_absorb_rejects_bad_args():
    lib = binding.lib()
    vp = ctypes.c_void_p
    p = _v3_params()
    assert lib.mla_absorb_q(None, vp(1), vp(1), vp(1), None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(ctypes.byref(p), vp(0), vp(0x1000), vp(0x2000), None) == \
        mla.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(ctypes.byref(_v3_params(dtype=5)), vp(0x1000), vp(0x1000),
                            vp(0x2000), None) == mla.MLA_ERR_UNSUPPORTED


def _prefill_params(**kw):
    base = dict(batch=1, tokens=4096, heads=128, d_c=512, d_r=64, d_n=128, d_v=128, n_max=4096,
                ckv_stride_b=4096 * 576, ckv_stride_n=576, kpe_stride_b=4096 * 576,
                kpe_stride_n=576, softmax_scale=0.0, dtype=mla.MLA_BF16, out_dtype=mla.MLA_BF16,
                num_splits=0, q_rope_base=0.0)
    base.update(kw)
    return binding.PrefillParams(**base)


def test_prefill_workspace_and_validation():
    p = _prefill_params()
    assert mla.prefill_workspace_bytes(p) == 2 * 4096 * 128 * 128 * 2
    assert mla.prefill_workspace_bytes(_prefill_params(q_rope_base=10000.0)) == \
        2 * 4096 * 128 * 128 * 2 + 4096 * 128 * 64 * 2                # + rotated q_rope
    assert mla.prefill_workspace_bytes(_prefill_params(tokens=5000)) == 0   # T > n_max
    assert mla.prefill_workspace_bytes(_prefill_params(num_splits=1)) == 0  # naive: no splits
    assert mla.prefill_workspace_bytes(_prefill_params(q_rope_base=0.5)) == 0
    lib = binding.lib()
    vp = ctypes.c_void_p
    args = [vp(0x1000)] * 8

    def call(pp, ws=0x100000, nbytes=1 << 40, ptrs=args):
        return lib.mla_prefill_naive(ctypes.byref(pp), *ptrs, vp(ws), nbytes, None)

    assert call(_prefill_params(d_c=128)) == mla.MLA_ERR_UNSUPPORTED
    assert call(_prefill_params(tokens=0)) == mla.MLA_ERR_INVALID_ARG
    assert call(p, nbytes=10) == mla.MLA_ERR_WORKSPACE
    assert call(p, ptrs=[vp(0)] + args[1:]) == mla.MLA_ERR_INVALID_ARG


def test_decode_num_splits_balanced_plan():
    # bf16, num_splits = 0: the smallest width C >= 4 tiles with at most 256
    # items in all, reported for sequences holding all n_max = 131072 rows
    # (4096 tiles of 32): B sequences get 256 / B items each while that
    # leaves C >= 4 and at most 256 per sequence.
    for batch, want in ((1, 256), (2, 128), (4, 64), (8, 32), (32, 8), (128, 2)):
        assert mla.decode_num_splits(_v3_params(batch=batch)) == want, batch
    # 200 sequences: 2 items each would be 400 > 256, so one each; likewise 300
    assert mla.decode_num_splits(_v3_params(batch=200)) == 1
    assert mla.decode_num_splits(_v3_params(batch=300)) == 1
    # 4096 rows (128 tiles) at batch 8: C = 4 -> 32 items per sequence
    short = dict(n_max=4096, ckv_stride_b=4096 * 576, kpe_stride_b=4096 * 576)
    assert mla.decode_num_splits(_v3_params(**short)) == 32
    # 64 rows (2 tiles): the 4-tile minimum keeps each sequence whole
    tiny = dict(n_max=64, ckv_stride_b=64 * 576, kpe_stride_b=64 * 576)
    assert mla.decode_num_splits(_v3_params(**tiny)) == 1
    # 3 sequences: 256 // 3 = 85 items at most -> C = ceil(4096 / 85) = 49 ->
    # 84 items per sequence (252 in all)
    assert mla.decode_num_splits(_v3_params(batch=3)) == 84
    # a fixed count is reported as set
    assert mla.decode_num_splits(_v3_params(num_splits=5)) == 5
    # the fp32 path picks one count from the sizes: 256 / (8 * 128) -> 1
    assert mla.decode_num_splits(_v3_params(dtype=mla.MLA_F32, out_dtype=mla.MLA_F32)) == 1


def test_prefill_absorbed_workspace_and_splits():
    T = 16
    p = _prefill_params(tokens=T, n_max=131072, ckv_stride_b=131072 * 576,
                        kpe_stride_b=131072 * 576, num_splits=4)
    rows = T * 128
    rnd = lambda x: (x + 255) // 256 * 256
    assert mla.prefill_absorbed_num_splits(p) == 4
    # q~ | q_rope, partials and (m, l) of 4 splits, and the merged latents of
    # the batched up-projection (query rows x heads = 2048 >= 1024)
    # and the plan's item table (16 query rows x 4 items of 16 bytes) and row
    # table (16 x 8 bytes)
    assert mla.prefill_absorbed_workspace_bytes(p) == \
        rnd(rows * 576 * 2) + rnd(rows * 4 * 512 * 4) + rnd(rows * 4 * 2 * 4) + \
        rnd(rows * 512 * 4) + rnd(T * 4 * 16) + rnd(T * 8)
    # auto split count: enough (query row, split) blocks for the chip
    auto = _prefill_params(tokens=T, n_max=131072, ckv_stride_b=131072 * 576,
                           kpe_stride_b=131072 * 576)
    assert mla.prefill_absorbed_num_splits(auto) == 16
    assert mla.prefill_absorbed_num_splits(_prefill_params()) == 1      # 4096 rows already
    assert mla.prefill_absorbed_workspace_bytes(_prefill_params(heads=96)) == 0
    assert mla.prefill_absorbed_workspace_bytes(_prefill_params(batch=20)) == 0  # B*T > 65535


@pytest.mark.parametrize("kw,status", [
    (dict(heads=96), "UNSUPPORTED"),
    (dict(d_c=128), "UNSUPPORTED"),
    (dict(batch=17), "UNSUPPORTED"),       # batch * tokens beyond 65535
    (dict(tokens=5000), "INVALID_ARG"),    # more queries than cache rows
    (dict(num_splits=-1), "INVALID_ARG"),
    (dict(num_splits=300), "INVALID_ARG"),
    (dict(q_rope_base=1.0), "INVALID_ARG"),
    (dict(softmax_scale=-1.0), "INVALID_ARG"),
    (dict(ckv_stride_n=1 << 50), "UNSUPPORTED"),   # n_max * stride beyond 64 bits
    (dict(kpe_stride_b=-8), "INVALID_ARG"),
])
def test_prefill_absorbed_rejects_bad_params_before_launch(kw, status):
    lib = binding.lib()
    vp = ctypes.c_void_p
    pp = _prefill_params(**kw)
    rc = lib.mla_prefill_absorbed(ctypes.byref(pp), *([vp(0x1000)] * 8), vp(0x100000), 1 << 40,
                                  None)
    assert rc == getattr(mla, "MLA_ERR_" + status)
    assert _msg() != ""


def test_prefill_absorbed_rejects_null_pointers_and_small_workspace():
    lib = binding.lib()
    vp = ctypes.c_void_p
    pp = _prefill_params(tokens=8, num_splits=2)
    ptrs = [vp(0x1000)] * 8
    for i in range(8):
        bad = list(ptrs)
        bad[i] = vp(0)
        assert lib.mla_prefill_absorbed(ctypes.byref(pp), *bad, vp(0x100000), 1 << 40,
                                        None) == mla.MLA_ERR_INVALID_ARG, i
    need = mla.prefill_absorbed_workspace_bytes(pp)
    assert lib.mla_prefill_absorbed(ctypes.byref(pp), *ptrs, vp(0x100000), need - 1,
                                    None) == mla.MLA_ERR_WORKSPACE


def _proj_params(**kw):
    base = dict(batch=8, in_features=16384, out_features=7168, dtype=mla.MLA_BF16,
                out_dtype=mla.MLA_BF16, num_splits=0, reserved=0)
    base.update(kw)
    return binding.ProjParams(**base)


def test_output_proj_workspace_and_validation():
    assert ctypes.sizeof(binding.ProjParams) == 3 * 8 + 4 * 4
    # auto, bf16, >= 2048 rows: the direct form, no workspace
    assert mla.output_proj_workspace_bytes(_proj_params()) == 0
    assert mla.output_proj_workspace_bytes(_proj_params(in_features=65536)) == 0
    # auto with fewer rows, or fp32: slices of ~1024 input features, fp32 partials of every slice
    assert mla.output_proj_workspace_bytes(_proj_params(out_features=2047)) == 16 * 8 * 2047 * 4
    assert mla.output_proj_workspace_bytes(_proj_params(dtype=mla.MLA_F32)) == 16 * 8 * 7168 * 4
    # an explicit split count always takes the sliced form
    assert mla.output_proj_workspace_bytes(_proj_params(num_splits=3)) == 3 * 8 * 7168 * 4
    assert mla.output_proj_workspace_bytes(_proj_params(in_features=100)) == 0   # bf16: K % 64
    assert mla.output_proj_workspace_bytes(_proj_params(in_features=100, dtype=mla.MLA_F32)) > 0
    lib = binding.lib()
    vp = ctypes.c_void_p
    for kw, status in [(dict(batch=0), "INVALID_ARG"), (dict(reserved=1), "INVALID_ARG"),
                       (dict(num_splits=-1), "INVALID_ARG"), (dict(dtype=9), "UNSUPPORTED"),
                       (dict(in_features=96), "UNSUPPORTED")]:
        pp = _proj_params(**kw)
        rc = lib.mla_output_proj(ctypes.byref(pp), vp(0x1000), vp(0x2000), vp(0x3000),
                                 vp(0x100000), 1 << 40, None)
        assert rc == getattr(mla, "MLA_ERR_" + status), kw
    pp = _proj_params()
    assert lib.mla_output_proj(ctypes.byref(pp), vp(0x1008), vp(0x2000), vp(0x3000),
                               vp(0x100000), 1 << 40, None) == mla.MLA_ERR_INVALID_ARG  # x % 16
    pp = _proj_params(num_splits=3)   # the sliced form, whose partials need a workspace
    assert lib.mla_output_proj(ctypes.byref(pp), vp(0x1000), vp(0x2000), vp(0x3000),
                               vp(0x100000), 100, None) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_output_proj(ctypes.byref(pp), vp(0x1000), vp(0x2000), vp(0x3000),
                               None, 1 << 40, None) == mla.MLA_ERR_WORKSPACE


def test_fold_and_decode_latent_reject_before_launch():
    lib = binding.lib()
    vp = ctypes.c_void_p
    f = lib.mla_fold_value_output
    assert f(0, 128, 128, 512, mla.MLA_BF16, vp(0x1000), vp(0x2000), vp(0x3000), None) == \
        mla.MLA_ERR_INVALID_ARG
    assert f(7168, 128, 128, 512, 5, vp(0x1000), vp(0x2000), vp(0x3000), None) == \
        mla.MLA_ERR_UNSUPPORTED
    assert f(7168, 128, 128, 512, mla.MLA_BF16, vp(0), vp(0x2000), vp(0x3000), None) == \
        mla.MLA_ERR_INVALID_ARG
    p = _v3_params(d_v=1)   # d_v is not used by the latent form
    d = lib.mla_decode_latent
    assert d(ctypes.byref(p), vp(0x1000), vp(0x2000), vp(0x3000), vp(0x5000), vp(0x5400),
             vp(0x6000), vp(0x7000), vp(0x100000), 10, None) == mla.MLA_ERR_WORKSPACE
    assert d(ctypes.byref(p), vp(0x1000), vp(0x2000), vp(0x3000), vp(0x5000), vp(0x5400),
             vp(0x6000), vp(0), vp(0x100000), 1 << 40, None) == mla.MLA_ERR_INVALID_ARG
    assert d(ctypes.byref(_v3_params(heads=96)), vp(0x1000), vp(0x2000), vp(0x3000), vp(0x5000),
             vp(0x5400), vp(0x6000), vp(0x7000), vp(0x100000), 1 << 40, None) == \
        mla.MLA_ERR_UNSUPPORTED


def _append_params(**kw):
    base = dict(batch=8, d_model=7168, d_c=512, d_r=64, n_max=4096, ckv_stride_b=4096 * 576,
                ckv_stride_n=576, kpe_stride_b=4096 * 576, kpe_stride_n=576, rope_base=0.0,
                dtype=mla.MLA_BF16, reserved=0)
    base.update(kw)
    return binding.AppendParams(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d_r=63), "UNSUPPORTED"),          # rotation pairs need an even width
    (dict(d_c=511), "UNSUPPORTED"),
    (dict(d_model=7170), "UNSUPPORTED"),    # not a whole number of 16-byte pieces
    (dict(dtype=7), "UNSUPPORTED"),
    (dict(reserved=1), "INVALID_ARG"),
    (dict(n_max=0), "INVALID_ARG"),
    (dict(ckv_stride_n=500), "INVALID_ARG"),
    (dict(ckv_stride_b=576), "INVALID_ARG"),
    (dict(rope_base=1.0), "INVALID_ARG"),
    (dict(rope_base=-5.0), "INVALID_ARG"),
    (dict(ckv_stride_n=1 << 52), "UNSUPPORTED"),   # n_max * stride beyond 64 bits
    (dict(kpe_stride_b=1 << 61), "UNSUPPORTED"),
])
def test_append_rejects_bad_params_before_launch(kw, status):
    lib = binding.lib()
    vp = ctypes.c_void_p
    p = _append_params(**kw)
    rc = lib.mla_cache_append(ctypes.byref(p), *[vp(0x1000)] * 6, None)
    assert rc == getattr(mla, "MLA_ERR_" + status)


def test_append_rejects_null_and_misaligned_pointers():
    lib = binding.lib()
    vp = ctypes.c_void_p
    p = _append_params()
    good = [vp(0x1000)] * 6
    for i in range(6):
        bad = list(good)
        bad[i] = vp(0)
        assert lib.mla_cache_append(ctypes.byref(p), *bad, None) == mla.MLA_ERR_INVALID_ARG
    bad = list(good)
    bad[0] = vp(0x1008)                  # h not 16-byte aligned
    assert lib.mla_cache_append(ctypes.byref(p), *bad, None) == mla.MLA_ERR_INVALID_ARG
    # an empty batch is a no-op that needs no pointers
    assert lib.mla_cache_append(ctypes.byref(_append_params(batch=0)), *[vp(0)] * 6, None) == 0


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-41, 65504.0, 1.0 + 2**-8 + 2**-20],
                 dtype=np.float32)
    bits = datagen.bf16_bits(x)
    back = datagen.bf16_to_f32(bits)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5
    assert back[6] == np.float32(1.0078125)  # just above the tie rounds up
    # every normal value is within half a bf16 ulp (8 significant bits)
    norm = np.abs(x) > 1e-37
    _, e = np.frexp(x[norm])
    half_ulp = np.ldexp(1.0, e - 9)
    assert np.all(np.abs(back[norm] - x[norm]) <= half_ulp)


def test_datagen_is_seeded_and_shaped():
    a = datagen.make_workload("tiny-f32")
    b = datagen.make_workload("tiny-f32")
    assert np.array_equal(a.cache, b.cache) and np.array_equal(a.w_uk, b.w_uk)
    assert a.cache.shape == (1, 128, 80) and a.dtype == "f32"
    assert a.scale == pytest.approx(1 / np.sqrt(48))
    c = datagen.make_decode_case(B=4, H=128, dc=512, dr=64, dn=128, dv=128, n_max=64,
                                 ragged=True, seed=3)
    assert c.cache.dtype == np.uint16 and c.cache.shape == (4, 64, 576)
    assert np.all((c.seqlens >= 1) & (c.seqlens <= 64))
    # weights have std 1/sqrt(d_c)
    w = datagen.bf16_to_f32(c.w_uk)
    assert abs(w.std() * np.sqrt(512) - 1) < 0.02


def test_binding_refuses_host_tensors_before_any_launch():
    """The binding passes plain pointers, so it checks every tensor first: host
    tensors are refused with MLA_ERR_INVALID_ARG and nothing reaches the GPU."""
    B, H, N = 2, 128, 64
    bf = torch.bfloat16
    cache = torch.zeros((B, N, 576), dtype=bf)
    args = (torch.zeros((B, H, 128), dtype=bf), torch.zeros((B, H, 64), dtype=bf),
            torch.zeros((H, 128, 512), dtype=bf), torch.zeros((H, 128, 512), dtype=bf),
            cache[:, :, :512], cache[:, :, 512:], torch.full((B,), N, dtype=torch.int32))
    with pytest.raises(mla.MLAError) as err:
        mla.decode(*args, workspace=None, out=torch.zeros((B, H, 128), dtype=bf))
    assert err.value.status == mla.MLA_ERR_INVALID_ARG and "GPU" in str(err.value)
    with pytest.raises(mla.MLAError) as err:
        mla.output_proj(torch.zeros((8, 16384), dtype=bf), torch.zeros((7168, 16384), dtype=bf),
                        out=torch.zeros((8, 7168), dtype=bf))
    assert err.value.status == mla.MLA_ERR_INVALID_ARG
    with pytest.raises(mla.MLAError) as err:
        mla.cache_append(torch.zeros((B, 7168), dtype=bf), torch.zeros((512, 7168), dtype=bf),
                         torch.zeros((64, 7168), dtype=bf), torch.zeros((B,), dtype=torch.int32),
                         cache[:, :, :512], cache[:, :, 512:])
    assert err.value.status == mla.MLA_ERR_INVALID_ARG
