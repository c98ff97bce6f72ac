"""CPU checks of the C ABI library: it loads, exports every symbol the header
declares, validates arguments before touching the GPU, and packs expert
blobs in the documented layout.  No kernel is launched."""
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return re.findall(r"^MOE_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def B():
    from int4_expert_ffn_int8_amd import binding
    binding.load()
    return binding


def test_library_exports_every_header_symbol(B):
    names = _header_functions()
    assert len(names) >= 10
    lib = B.load()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_blob_bytes_match_layout(B):
    # 35B-shaped expert: codes 1,572,864 + scale/bias 196,608 + LoRA 245,760
    assert B.moe_expert_blob_bytes(2048, 512, 16) == 2015232 + 256  # sections + the 256-byte meta
    assert B.moe_expert_blob_bytes(256, 128, 4) == 64512 + 256
    assert B.moe_expert_blob_bytes(2000, 512, 16) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(H=2000), 1), (dict(K=0), 1), (dict(K=300), 1), (dict(r=17), 2), (dict(E=2000), 2),
    (dict(n_shared=2), 1), (dict(norm_topk=3), 1), (dict(H=8192), 2),
])
def test_route_rejects_bad_dims_without_launch(B, bad, code):
    p = dict(H=2048, I=512, E=256, K=4, r=16, n_shared=1, norm_topk=1)
    p.update(bad)
    d = B.MoeDims(p["H"], p["I"], p["E"], p["K"], p["r"], p["n_shared"], p["norm_topk"], 1.0)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(d, None, None, None, None, None, 1, None, None, None, None, None, None, None,
                    None, None, stream=0)
    assert ei.value.status == code, str(ei.value)


def test_route_null_pointers_and_workspace(B):
    d = B.dims(2048, 512, 256, 4, 16, 1)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(d, None, None, None, None, None, 1, None, None, None, None, None, None, None,
                    None, None, stream=0)
    assert ei.value.status == 1
    # fake non-null addresses: the workspace check fires before any launch
    fake = 1 << 40
    with pytest.raises(B.MoeError) as ei:
        B.load().moe_route(B.ctypes.byref(d), fake, fake, fake, fake, fake, 1, None, fake, fake,
                           fake, None, None, None, None, fake, 16, 0)
        B._check(1)
    assert "workspace" in str(ei.value)
    # partial grouping outputs are rejected
    st = B.load().moe_route(B.ctypes.byref(d), fake, fake, fake, fake, fake, 1, None, fake, fake,
                            fake, None, fake, None, None, fake, 1 << 30, 0)
    assert st == 1
    # T == 0 is a no-op
    assert B.load().moe_route(B.ctypes.byref(d), None, None, None, None, None, 0, None, None,
                              None, None, None, None, None, None, None, 0, 0) == 0


def test_block_prefill_validation_and_workspace(B):
    # every check of moe_block_prefill fires before any device work
    d = B.dims(2048, 512, 256, 4, 16, 1)
    lib = B.load()
    T = 3300
    need = lib.moe_block_prefill_workspace_bytes(B.ctypes.byref(d), T)
    base = B.moe_workspace_bytes(d, T, True)
    # the route + expert workspace, then counts, offsets, perm, shared gate,
    # the compact expert outputs (fp16) and one exponent per (token, slot) row
    assert need >= base + T * 5 * 2048 * 2 + T * 5 * 4 + T * 4 * 4
    assert lib.moe_block_prefill_workspace_bytes(B.ctypes.byref(B.dims(2000, 512, 256, 4, 16, 1)), 1) == 0
    fake = 1 << 40
    ex = B.MoeExperts(fake, 256, None, None, None, 0)
    args = lambda x, T, ws, nbytes, eps=1e-6: (B.ctypes.byref(d), fake, fake, fake, fake, None,
                                               B.ctypes.byref(ex), fake, x, T, None, fake, fake,
                                               fake, None, eps, ws, nbytes, 0)
    assert lib.moe_block_prefill(*args(None, 0, None, 0)) == 0          # T == 0: nothing to do
    assert lib.moe_block_prefill(*args(fake, -1, fake, need)) == 1      # negative T
    assert lib.moe_block_prefill(*args(None, T, fake, need)) == 1       # null x
    st = lib.moe_block_prefill(*args(fake, T, fake, need - 1))          # short workspace
    assert st != 0 and "workspace" in lib.moe_last_error().decode()
    d2 = B.dims(2048, 512, 256, 4, 16, 1)
    nout = (B.ctypes.byref(d2), fake, fake, fake, fake, None, B.ctypes.byref(ex), fake, fake, T,
            None, fake, fake, fake, fake, float("nan"), fake, need, 0)
    assert lib.moe_block_prefill(*nout) == 1                            # norm output with a NaN eps


def test_expert_forward_validation(B):
    d = B.dims(2048, 512, 256, 4, 16, 1)
    fake = 1 << 40
    few = B.experts_struct(fake, 64)  # no table but only 64 slots
    st = B.load().moe_expert_forward(B.ctypes.byref(d), B.ctypes.byref(few), fake, fake, 1, fake,
                                     None, None, None, fake, fake, 1 << 30, 0)
    assert st == 1 and b"cover" in B.load().moe_last_error()
    tab = B.experts_struct(fake, 64, expert_to_slot=fake)  # table but no host copy
    st = B.load().moe_expert_forward(B.ctypes.byref(d), B.ctypes.byref(tab), fake, fake, 1, fake,
                                     None, None, None, fake, fake, 1 << 30, 0)
    assert st == 1 and b"host_blobs" in B.load().moe_last_error()
    full = B.experts_struct(fake, 256)
    st = B.load().moe_expert_forward(B.ctypes.byref(d), B.ctypes.byref(full), None, fake, 1, fake,
                                     None, None, None, fake, fake, 1 << 30, 0)
    assert st == 1 and b"shared_blob" in B.load().moe_last_error()


def test_block_decode_exec_and_read_delay_validation(B):
    # checked on the host before any launch: a NULL exec_idx, and a modeled
    # read latency above MOE_MAX_READ_DELAY_NS (1 ms)
    d = B.dims(2048, 512, 256, 4, 16, 1)
    fake = 1 << 40
    lib = B.load()
    tab = B.experts_struct(fake, 64, expert_to_slot=fake, host_blobs=fake)
    st = lib.moe_block_decode_exec(B.ctypes.byref(d), fake, fake, fake, fake, B.ctypes.byref(tab),
                                   fake, fake, 1, 0, 0.0, None, None, None, fake, fake, 1 << 30, 0)
    assert st == 1 and b"exec_idx" in lib.moe_last_error()
    slow = B.experts_struct(fake, 64, expert_to_slot=fake, host_blobs=fake,
                            read_delay_ns=1_000_001)
    for call in ("moe_block_decode", "moe_block_decode_exec"):
        args = [B.ctypes.byref(d), fake, fake, fake, fake, B.ctypes.byref(slow), fake, fake, 1, 0,
                0.0]
        if call == "moe_block_decode_exec":
            args.append(fake)
        args += [None, None, fake, fake, 1 << 30, 0]
        st = getattr(lib, call)(*args)
        assert st == 1 and b"read_delay_ns" in lib.moe_last_error(), call
    # T == 0 with no exec_idx is a no-op
    ok = B.experts_struct(fake, 256)
    assert lib.moe_block_decode_exec(B.ctypes.byref(d), fake, fake, fake, fake, B.ctypes.byref(ok),
                                     fake, fake, 0, 0, 0.0, None, None, None, fake, fake, 1 << 30,
                                     0) == 0
    assert lib.moe_pool_set_read_delay(None, 0) == 1


def test_prerouter_validation(B):
    fake = 1 << 40
    assert B.load().prerouter_predict(fake, fake, 2048, 256, 256, 0, fake, 1, fake, None, fake,
                                      1 << 20, 0) == 1
    assert B.load().prerouter_predict(fake, fake, 2048, 100, 256, 4, fake, 1, fake, None, fake,
                                      1 << 20, 0) == 1
    assert B.load().prerouter_predict(fake, fake, 2048, 256, 256, 4, fake, 1, fake, None, fake,
                                      16, 0) == 4
    # features: W1 rows of H + E columns must be 16-byte multiples
    assert B.load().prerouter_predict_feat(fake, fake, 2048, 256, 100, 4, fake, fake, 4, 1, fake,
                                           None, fake, 1 << 20, 0) == 2
    assert B.load().prerouter_predict(fake, fake, 2048, 256, 256, 4, fake, 1 << 16, fake, None,
                                      fake, 1 << 40, 0) == 2
    # the workspace holds the launch counter and the partial logits of ceil(D / 8)
    # row blocks per token, as 8-byte hand-off words
    assert B.prerouter_workspace_bytes(256, 256, 1) >= 256 + 32 * 256 * 8
    assert B.prerouter_workspace_bytes(4096, 1000, 3) >= 256 + 3 * 512 * 1000 * 8


def _unpack_codes(rows_bytes, n):
    """Decode packed code rows with the documented nibble order:
    word w holds columns 8w+2s in bits [4s,4s+4) and 8w+2s+1 in [16+4s, 20+4s)."""
    words = rows_bytes.view(np.uint32)
    out = np.zeros((words.shape[0], n), np.uint8)
    for s in range(4):
        out[:, 2 * s::8] = (words >> (4 * s)) & 0xF
        out[:, 2 * s + 1::8] = (words >> (16 + 4 * s)) & 0xF
    return out


def test_pack_expert_layout_round_trip(B):
    w = synth.workload(0)
    H, I, r = w["H"], w["I"], w["r"]
    ex = synth.expert_tensors(w, 0, 3)
    blob = np.zeros(B.moe_expert_blob_bytes(H, I, r), np.uint8)
    B.moe_pack_expert(H, I, r, ex, blob)

    def a256(v):
        return (v + 255) // 256 * 256
    o = 0
    sec = {}
    for name, size in [("gu_codes", 2 * I * H // 2), ("gu_sb", 2 * I * (H // 64) * 4),
                       ("dn_codes", H * I // 2), ("dn_sb", H * (I // 64) * 4),
                       ("a_gu", 2 * r * H * 2), ("b_gu", 2 * I * r * 2), ("a_dn", r * I * 2),
                       ("b_dn", H * r * 2), ("meta", 8)]:
        sec[name] = blob[o:o + size]
        o = a256(o + size)
    assert o == blob.size
    gu = _unpack_codes(sec["gu_codes"].reshape(2 * I, H // 2), H)
    gu_sb = sec["gu_sb"].view(np.uint32).reshape(2 * I, H // 64)
    b_gu = sec["b_gu"].view(np.uint16).reshape(2 * I, r)
    for j in range(I):
        rg = (j // 16) * 32 + j % 16
        ru = rg + 16
        assert np.array_equal(gu[rg], ex["q_gate"][j]) and np.array_equal(gu[ru], ex["q_up"][j])
        assert np.array_equal(gu_sb[rg] & 0xFFFF, ex["s_gate"][j])
        assert np.array_equal(gu_sb[rg] >> 16, ex["b_gate"][j])
        assert np.array_equal(gu_sb[ru] & 0xFFFF, ex["s_up"][j])
        assert np.array_equal(b_gu[rg], ex["B_gate"][j]) and np.array_equal(b_gu[ru], ex["B_up"][j])
    dn = _unpack_codes(sec["dn_codes"].reshape(H, I // 2), I)
    assert np.array_equal(dn, ex["q_down"])
    dn_sb = sec["dn_sb"].view(np.uint32).reshape(H, I // 64)
    assert np.array_equal(dn_sb >> 16, ex["b_down"])
    a_gu = sec["a_gu"].view(np.uint16).reshape(2, r, H)
    assert np.array_equal(a_gu[0], ex["A_gate"]) and np.array_equal(a_gu[1], ex["A_up"])
    assert np.array_equal(sec["a_dn"].view(np.uint16).reshape(r, I), ex["A_down"])
    assert np.array_equal(sec["b_dn"].view(np.uint16).reshape(H, r), ex["B_down"])
    # meta: bounds of the down projection's outputs, from their definition
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # bf16 bits
    wd = f(ex["s_down"]).repeat(64, axis=1) * ex["q_down"] + f(ex["b_down"]).repeat(64, axis=1)
    w_bound = np.abs(wd).sum(axis=1).max()
    l_bound = (np.abs(f(ex["B_down"])) @ np.abs(f(ex["A_down"])).sum(axis=1)).max()
    meta = sec["meta"].view(np.float32)
    assert w_bound <= meta[0] <= w_bound * (1 + 1e-5)
    assert l_bound <= meta[1] <= l_bound * (1 + 1e-5)
    # the bound holds: |deq(Q_d) h + B_d (A_d h)| <= (W + L) max|h| for any h
    h = np.random.default_rng(0).standard_normal(I)
    y = wd @ h + f(ex["B_down"]) @ (f(ex["A_down"]) @ h)
    assert np.abs(y).max() <= (meta[0] + meta[1]) * np.abs(h).max()


def test_pack_rejects_codes_above_15(B):
    w = synth.workload(0)
    ex = synth.expert_tensors(w, 0, 0)
    ex["q_down"] = ex["q_down"].copy()
    ex["q_down"][5, 7] = 16
    blob = np.zeros(B.moe_expert_blob_bytes(w["H"], w["I"], w["r"]), np.uint8)
    with pytest.raises(B.MoeError):
        B.moe_pack_expert(w["H"], w["I"], w["r"], ex, blob)


@pytest.mark.parametrize("proj,s,b,ok", [
    ("gate", 4000.0, 0.0, True),        # 15 s = 60000: inside fp16
    ("gate", 4400.0, 0.0, False),       # 15 s = 66000: beyond fp16
    ("up", 1.0, -65280.0, True),        # |b| the largest bf16 inside fp16, 15 s + b inside
    ("down", 2.0, 65500.0, False),      # 15 s + b beyond fp16
    ("down", float("nan"), 0.0, False),
    ("up", 0.0, float("inf"), False),
])
def test_pack_rejects_groups_outside_f16_range(B, proj, s, b, ok):
    # the prefill GEMMs dequantise w = fp16(s q + b); the packer refuses
    # groups whose weights fp16 cannot hold
    w = synth.workload(0)
    ex = synth.expert_tensors(w, 0, 0)
    for k, v in ((f"s_{proj}", s), (f"b_{proj}", b)):
        ex[k] = ex[k].copy()
        ex[k][3, 1] = synth.f32_to_bf16_bits(np.array([v], np.float32))[0] if np.isfinite(v) else (
            0x7FC0 if np.isnan(v) else 0x7F80)
    blob = np.zeros(B.moe_expert_blob_bytes(w["H"], w["I"], w["r"]), np.uint8)
    if ok:
        B.moe_pack_expert(w["H"], w["I"], w["r"], ex, blob)
    else:
        with pytest.raises(B.MoeError) as ei:
            B.moe_pack_expert(w["H"], w["I"], w["r"], ex, blob)
        assert ei.value.status == 2 and "fp16" in str(ei.value)


def test_block_decode_noalloc_validates_before_device_work(B):
    # the allocation-free decode entry point checks its arguments before it
    # looks up or touches its device scratch: no GPU is needed for these
    lib = B.load()
    fake = 1 << 40
    ex = B.experts_struct(fake, 256)
    d = B.dims(2048, 512, 256, 4, 16, 1)
    args = lambda T, dd=d, flags=0: (B.ctypes.byref(dd), fake, fake, fake, fake,
                                     B.ctypes.byref(ex), fake, fake, T, flags, 1e-6, None, None,
                                     fake, None, 0)
    assert lib.moe_block_decode_noalloc(*args(0)) == 0          # T == 0: no-op
    assert lib.moe_block_decode_noalloc(*args(2)) == 2          # 10 pairs > 8
    assert lib.moe_block_decode_noalloc(*args(-1)) == 1
    assert lib.moe_block_decode_noalloc(*args(1, flags=8)) == 1
    assert lib.moe_block_decode_noalloc(*args(1, dd=B.dims(2048, 512, 256, 4, 17, 1))) == 2
    assert b"noalloc" in lib.moe_last_error()


def test_noalloc_scratch_holds_every_supported_fused_shape(B):
    # the allocation-free decode's scratch (MOE_NOALLOC_SCRATCH_BYTES) holds
    # the fused workspace of the largest supported shapes: 8 (token, slot)
    # pairs, I = 2048, r = 16, and 4 tokens over 1024 experts
    import re
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    cap = int(re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES (\d+)", hdr).group(1))
    worst = 0
    for T, K, S in [(4, 1, 1), (1, 8, 0), (2, 3, 1), (1, 7, 1), (4, 2, 0)]:
        for E in (K, 256, 1024):
            d = B.dims(2048, 2048, E, K, 16, S)
            n = int(B.load().moe_block_decode_workspace_bytes(B.ctypes.byref(d), T))
            assert n > 0
            worst = max(worst, n)
    assert worst <= cap, (worst, cap)
