"""Host-side checks of libtilemix through its C ABI (no GPU needed): exported
symbols, routing words bit-exact with the oracle, the work plan, and argument
validation."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import mixed_precision_attention_amd as tm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tilemix.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tm.LIB_PATH),
                                reason="libtilemix.so not built (run __graft_entry__.build())")


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(tilemix_[a-z0-9_]+)\s*\(", text)))
    assert len(names) >= 8
    lib = ctypes.CDLL(tm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


PROBES_LIB = os.path.join(os.path.dirname(tm.LIB_PATH), "libtilemix_probes.so")


@pytest.mark.skipif(not os.path.exists(PROBES_LIB), reason="libtilemix_probes.so not built")
def test_probe_library_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "tilemix_probes.h")).read()
    names = sorted(set(re.findall(r"\b(tilemix_probe_[a-z0-9_]+)\s*\(", text)))
    assert len(names) == 7
    lib = ctypes.CDLL(PROBES_LIB)
    for n in names:
        assert hasattr(lib, n), n
    # the attention library exports none of them
    main = ctypes.CDLL(tm.LIB_PATH)
    assert not any(hasattr(main, n) for n in names)


@pytest.mark.parametrize("template", oracle.TEMPLATES)
def test_routing_bit_exact_with_oracle(template):
    for lens in ([256], [1], [130], [1000], [4096], [8192], [300, 0, 77, 129, 2049],
                 [16384, 1024]):
        for cov in (0, 1000, 2500, 5000, 7500, 10000):
            for seed in (0, 12345):
                w, g, n8, nl = tm.tilemix_build_routing(synth.cu_seqlens_of(lens), 3, template, cov, seed)
                ow, og, on8, onl = oracle.routing_words(lens, 3, template, cov, seed)
                assert np.array_equal(w, ow), (lens, cov, seed)
                assert np.array_equal(g, og) and np.array_equal(n8, on8) and np.array_equal(nl, onl)


def test_routing_large_varlen_matches_oracle():
    lens = synth.WORKLOADS["qwen2_7b_varlen"]["seqlens"]
    w, g, n8, nl = tm.tilemix_build_routing(synth.cu_seqlens_of(lens), 4, "rowrandom", 5000, 0)
    ow, og, on8, onl = oracle.routing_words(lens, 4, "rowrandom", 5000, 0)
    assert np.array_equal(w, ow) and list(n8) == [8320, 2080, 1040, 528, 36, 36]


def test_query_sizes():
    t, tq, tk = tm.tilemix_query_sizes([0, 256, 256, 386])
    assert (t, tq, tk) == (386, 2 + 0 + 2, 4 + 0 + 3)


def _plan_parts(plan):
    hdr = plan[:16]
    batch, hq, hkv = hdr[2], hdr[3], hdr[4]
    seqtab = plan[hdr[10]:hdr[10] + 8 * batch].reshape(batch, 8)
    items = plan[hdr[11]:hdr[11] + 2 * hdr[9]].reshape(-1, 2)
    return hdr, seqtab, items


@pytest.mark.parametrize("lens,hq,hkv", [([4096] * 8, 24, 8), ([65536, 16384, 8192, 4096, 1024, 1024], 28, 4),
                                         ([300, 0, 77, 129, 1], 6, 2), ([256], 1, 1)])
def test_plan_covers_every_unit_once(lens, hq, hkv):
    cu = synth.cu_seqlens_of(lens)
    plan = tm.tilemix_build_plan(cu, hq, hkv, 128)
    hdr, seqtab, items = _plan_parts(plan)
    assert hdr[0] == 0x544D5850 and hdr[6] == cu[-1]
    qt = kt = 0
    for s, L in enumerate(lens):
        geo = oracle.seq_geometry(L)
        assert list(seqtab[s][:7]) == [cu[s], L, qt, kt, geo.g, geo.Tm, geo.Tn]
        qt += geo.Tm
        kt += geo.Tn
    assert (hdr[7], hdr[8]) == (qt, kt)
    real = [(int(a), int(b) >> 16, int(b) & 0xffff) for a, b in items if a >= 0]
    expect = {(s, h, r) for s, L in enumerate(lens) for h in range(hq)
              for r in range(oracle.seq_geometry(L).Tm)}
    assert len(real) == len(expect) and set(real) == expect
    # units sharing a (sequence, KV head) are dealt to few dies, in runs that
    # stay contiguous in the die's queue; each run goes longest row first
    die = {}
    for pos, (a, b) in enumerate(items):
        if a < 0:
            continue
        h, r = int(b) >> 16, int(b) & 0xffff
        geo = oracle.seq_geometry(lens[a])
        die.setdefault(pos % 8, []).append(((int(a), h // (hq // hkv)), geo.last_tile[r] + 1))
    groups_per_die = []
    for q in die.values():
        runs = [[q[0]]]
        for x in q[1:]:
            if x[0] == runs[-1][-1][0] and x[1] <= runs[-1][-1][1]:
                runs[-1].append(x)
            else:
                runs.append([x])
        # a group appears in few runs (it is split only when larger than
        # half a die's share)
        keys = [r[0][0] for r in runs]
        assert len(keys) <= 2 * len(set(keys))
        groups_per_die.append(len(set(keys)))
    assert max(groups_per_die) <= max(1, -(-len(lens) * hkv // 8)) + 2


def test_errors_are_reported():
    cu = synth.cu_seqlens_of([256])
    with pytest.raises(tm.TileMixError, match="coverage_bp"):
        tm.tilemix_build_routing(cu, 1, "band", 10001)
    with pytest.raises(tm.TileMixError, match="template"):
        tm.tilemix_build_routing(cu, 1, 9, 100)
    with pytest.raises(tm.TileMixError, match="non-decreasing"):
        tm.tilemix_build_routing([0, 10, 5], 1, "band", 100)
    with pytest.raises(tm.TileMixError, match="cu_seqlens\\[0\\]"):
        tm.tilemix_query_sizes([3, 10])
    with pytest.raises(tm.TileMixError, match="Hq"):
        tm.tilemix_build_plan(cu, 5, 2, 128)
    with pytest.raises(tm.TileMixError, match="head_dim") as e:
        tm.tilemix_build_plan(cu, 2, 2, 96)
    assert e.value.code == -2
    lib = tm.lib()
    plan = tm.tilemix_build_plan(cu, 2, 1, 64)
    p = ctypes.c_void_p(plan.ctypes.data)
    fake = ctypes.c_void_p(16)
    odd = ctypes.c_void_p(24)
    # pointer validation happens before any device work
    assert lib.tilemix_quantize_qk(p, None, fake, fake, fake, fake, fake, fake, None) == -1
    assert "plan_d" in tm.tilemix_last_error()
    assert lib.tilemix_prefill_varlen(p, fake, fake, fake, fake, fake, odd, fake, fake, fake, fake, None) == -1
    assert "aligned" in tm.tilemix_last_error()
    bad = plan.copy()
    bad[0] = 7
    assert lib.tilemix_prefill_varlen(ctypes.c_void_p(bad.ctypes.data), fake, fake, fake, fake, fake, fake,
                                      fake, fake, fake, fake, None) == -1
    assert "not a TileMix plan" in tm.tilemix_last_error()
    assert lib.tilemix_quantize_k(p, fake, fake, odd, fake, None) == -1
    assert "k_i8" in tm.tilemix_last_error() and "aligned" in tm.tilemix_last_error()
    assert lib.tilemix_prefill_varlen_qinline(p, fake, fake, fake, fake, fake, None, fake, fake, None) == -1
    assert "k_scale is NULL" in tm.tilemix_last_error()
    assert lib.tilemix_debug_qk_i32_tile(p, fake, fake, fake, 0, 0, 5, 0, fake, None) == -1
    assert "row" in tm.tilemix_last_error()
    bad = plan.copy()
    bad[1] = 99
    assert lib.tilemix_quantize_qk(ctypes.c_void_p(bad.ctypes.data), fake, fake, fake, fake, fake, fake, fake,
                                   None) == -2


@pytest.mark.parametrize("template", oracle.TEMPLATES)
def test_three_class_routing_bit_exact_with_oracle(template):
    for lens in ([256], [1024, 300, 1, 0, 4160]):
        cu = synth.cu_seqlens_of(lens)
        for c8, cf in [(0, 0), (2500, 2500), (5000, 5000), (0, 10000), (7500, 2500), (1000, 0)]:
            got = tm.tilemix_build_routing3(cu, 2, template, c8, cf, 3)
            want = oracle.routing_words3(lens, 2, template, c8, cf, 3)
            assert all(np.array_equal(x, y) for x, y in zip(got, want)), (lens, c8, cf)
    with pytest.raises(tm.TileMixError, match="int8_bp"):
        tm.tilemix_build_routing3(synth.cu_seqlens_of([256]), 1, template, 6000, 5000)


@pytest.mark.parametrize("lens,hkv", [([256], 1), ([1024, 300, 1, 0, 129], 3), ([4160, 8192], 2)])
def test_adaptive_routing_bit_exact_with_oracle(lens, hkv):
    geos = [oracle.seq_geometry(L) for L in lens]
    rng = np.random.default_rng(len(lens))
    tm_total = sum(g.Tm for g in geos)
    imp = np.full((hkv, tm_total, 64), np.inf, dtype=np.float32)
    off = 0
    for geo in geos:
        for r in range(geo.Tm):
            # few distinct values, so ties (broken by (r, G)) are common
            imp[:, off + r, :geo.D[r] + 1] = -rng.integers(0, 4, size=(hkv, geo.D[r] + 1)) * np.float32(0.5)
        off += geo.Tm
    cu = synth.cu_seqlens_of(lens)
    for cov in (0, 1000, 2500, 5000, 7500, 10000):
        w, g, n8, nl = tm.tilemix_build_routing_adaptive(cu, imp, cov)
        ow, og, on8, onl = oracle.adaptive_words(lens, imp, cov)
        assert np.array_equal(w, ow), cov
        assert np.array_equal(g, og) and np.array_equal(n8, on8) and np.array_equal(nl, onl)
    bad = imp.copy()
    bad[0, 0, 0] = np.nan
    with pytest.raises(tm.TileMixError, match="NaN"):
        tm.tilemix_build_routing_adaptive(cu, bad, 5000)


def test_importance_host_checks():
    cu = synth.cu_seqlens_of([300, 0, 4096])
    plan = tm.tilemix_build_plan(cu, 6, 2, 128)
    _, tq, tk = tm.tilemix_query_sizes(cu)
    assert tm.tilemix_importance_workspace_size(plan) == (6 * tq + 2 * tk) * 128 * 4
    lib = tm.lib()
    p = ctypes.c_void_p(plan.ctypes.data)
    fake = ctypes.c_void_p(16)
    assert lib.tilemix_routing_importance(p, fake, fake, fake, fake, fake, fake, 100, fake, None) == -1
    assert "workspace" in tm.tilemix_last_error()
    long_plan = tm.tilemix_build_plan(synth.cu_seqlens_of([262145]), 1, 1, 64)
    assert lib.tilemix_routing_importance(ctypes.c_void_p(long_plan.ctypes.data), fake, fake, fake, fake,
                                          fake, fake, 1 << 40, fake, None) == -2


def test_decode_host_checks():
    cu = synth.cu_seqlens_of([300, 0, 4096])
    plan = tm.tilemix_build_plan(cu, 6, 2, 128)
    # B * Hq * ceil(max L / 256) * (d + 2) * 4 bytes
    assert tm.tilemix_decode_workspace_size(plan) == 3 * 6 * 16 * 130 * 4
    lib = tm.lib()
    p = ctypes.c_void_p(plan.ctypes.data)
    fake = ctypes.c_void_p(16)
    args = [p, fake, fake, fake, fake, fake, fake, fake, fake]
    assert lib.tilemix_decode_varlen(*args, 100, fake, None) == -1
    assert "workspace" in tm.tilemix_last_error()
    assert lib.tilemix_decode_varlen(p, fake, ctypes.c_void_p(24), *args[3:], 1 << 20, fake, None) == -1
    assert "aligned" in tm.tilemix_last_error()
    assert lib.tilemix_quantize_kv(p, fake, None, fake, fake, fake, fake, fake, None) == -1
    assert "k_f16" in tm.tilemix_last_error()
    empty = tm.tilemix_build_plan(np.array([0], dtype=np.int32), 2, 2, 64)
    pe = ctypes.c_void_p(empty.ctypes.data)
    assert tm.tilemix_decode_workspace_size(empty) == 0
    assert lib.tilemix_decode_varlen(pe, fake, None, None, None, None, None, None, None, 0, None, None) == 0


def test_empty_batch_is_a_no_op():
    cu = np.array([0, 0], dtype=np.int32)
    w, g, n8, nl = tm.tilemix_build_routing(cu, 2, "band", 5000)
    assert w.shape == (2, 0) and list(nl) == [0]
    plan = tm.tilemix_build_plan(cu, 2, 2, 64)
    lib = tm.lib()
    p = ctypes.c_void_p(plan.ctypes.data)
    fake = ctypes.c_void_p(16)
    # nothing to launch: returns OK without touching device pointers
    assert lib.tilemix_prefill_varlen(p, fake, None, None, None, None, None, None, None, None, None, None) == 0
    assert lib.tilemix_quantize_qk(p, fake, None, None, None, None, None, None, None) == 0
    assert lib.tilemix_quantize_k(p, fake, None, None, None, None) == 0
    assert lib.tilemix_prefill_varlen_qinline(p, fake, None, None, None, None, None, None, None, None) == 0


# ------------------------------------------------------- multi-layer stack

def test_stack_workspace_size():
    lens, hq, hkv, d = [300, 0, 77, 129, 1], 6, 2, 64
    cu = synth.cu_seqlens_of(lens)
    plan = tm.tilemix_build_plan(cu, hq, hkv, d)
    T, tq, tk = tm.tilemix_query_sizes(cu)

    def a256(n):
        return -(-n // 256) * 256
    # fp16 staging for (norm out / attention out), Q, K, V; K's codes and scales
    want = 2 * a256(T * hq * d * 2) + 2 * a256(T * hkv * d * 2) + a256(T * hkv * d) + a256(hkv * tk * 4)
    assert tm.tilemix_stack_workspace_size(plan) == want


def test_stack_argument_validation():
    lib = tm.lib()
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails validation first
    # empty input: nothing to do, no pointer needed
    assert lib.tilemix_stack_rms_norm(None, None, 0, 4, 2, 64, 1e-6, None) == 0
    assert lib.tilemix_stack_qkv(None, None, None, None, None, 0, 4, 2, 128, None) == 0
    assert lib.tilemix_stack_out_residual(None, None, None, 0, 4, 2, 64, None) == 0
    cases = [
        (lib.tilemix_stack_rms_norm, (fake, fake, 10, 4, 2, 96, 1e-6, None), -2, "head_dim"),
        (lib.tilemix_stack_rms_norm, (fake, fake, 10, 5, 2, 64, 1e-6, None), -1, "multiple"),
        (lib.tilemix_stack_rms_norm, (fake, fake, 10, 34, 2, 64, 1e-6, None), -2, "exceeds 1024"),
        (lib.tilemix_stack_rms_norm, (fake, fake, -1, 4, 2, 64, 1e-6, None), -1, "negative"),
        (lib.tilemix_stack_rms_norm, (fake, fake, 10, 4, 2, 64, -1.0, None), -1, "eps"),
        (lib.tilemix_stack_rms_norm, (None, fake, 10, 4, 2, 64, 1e-6, None), -1, "x is NULL"),
        (lib.tilemix_stack_rms_norm, (fake, P(0x1002), 10, 4, 2, 64, 1e-6, None), -1, "aligned"),
        (lib.tilemix_stack_qkv, (fake, fake, fake, None, fake, 10, 4, 2, 64, None), -1, "k_f16 is NULL"),
        (lib.tilemix_stack_out_residual, (fake, None, fake, 10, 4, 2, 64, None), -1, "wo_f16 is NULL"),
        (lib.tilemix_stack_qkv, (fake, fake, fake, fake, fake, 128 * 65536, 4, 2, 64, None), -1, "tokens"),
    ]
    for fn, args, code, text in cases:
        assert fn(*args) == code, text
        assert text in tm.tilemix_last_error(), (text, tm.tilemix_last_error())
    cu = synth.cu_seqlens_of([300, 20])
    plan = tm.tilemix_build_plan(cu, 4, 2, 64)
    need = tm.tilemix_stack_workspace_size(plan)
    rc = lib.tilemix_stack_layer(tm._hptr(plan), fake, fake, fake, fake, fake, 1e-6, fake, need - 1, None)
    assert rc == -1 and "workspace" in tm.tilemix_last_error()


def test_three_path_inline_entry_validation():
    cu = synth.cu_seqlens_of([200, 70])
    plan = tm.tilemix_build_plan(cu, 2, 1, 64)
    lib = tm.lib()
    p = ctypes.c_void_p(plan.ctypes.data)
    fake = ctypes.c_void_p(16)
    odd = ctypes.c_void_p(24)
    assert lib.tilemix_quantize_k_fp8(p, fake, fake, fake, None, None) == -1
    assert "k_scale_f8 is NULL" in tm.tilemix_last_error()
    assert lib.tilemix_quantize_k_i8_fp8(p, fake, fake, fake, fake, odd, fake, None) == -1
    assert "k_f8" in tm.tilemix_last_error() and "aligned" in tm.tilemix_last_error()
    assert lib.tilemix_prefill_varlen3_qinline(p, fake, fake, fake, fake, fake, fake, odd, fake, fake, fake,
                                               fake, None) == -1
    assert "k_f8" in tm.tilemix_last_error() and "aligned" in tm.tilemix_last_error()
    empty = tm.tilemix_build_plan(np.array([0, 0], dtype=np.int32), 2, 1, 64)
    e = ctypes.c_void_p(empty.ctypes.data)
    assert lib.tilemix_quantize_k_fp8(e, fake, None, None, None, None) == 0
    assert lib.tilemix_quantize_k_i8_fp8(e, fake, None, None, None, None, None, None) == 0
    assert lib.tilemix_prefill_varlen3_qinline(e, fake, *([None] * 10), None) == 0


def test_decode_noalloc_rejects_oversized_step_on_the_host():
    """The allocation-free decode step refuses, before any HIP call, a step
    whose partial records exceed its static scratch (fake device pointers:
    nothing is dereferenced on that path)."""
    lens = [65600, 1, 1, 1]
    plan_h = tm.tilemix_build_plan(synth.cu_seqlens_of(lens), 64, 8, 128)
    assert tm.tilemix_decode_workspace_size(plan_h) > 32 * 1024 * 1024
    fake = ctypes.c_void_p(1 << 20)
    rc = tm.lib().tilemix_decode_varlen_noalloc(plan_h.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, fake,
                                               fake, fake, fake, fake, None)
    assert rc == -1
    assert "scratch" in tm.tilemix_last_error()


def test_binding_refuses_tensors_smaller_than_the_plan():
    """The binding checks every tensor against the plan before any launch (CPU
    tensors: a wrong size is reported before the device check), and a device
    plan whose length differs from plan_h's."""
    torch = pytest.importorskip("torch")
    cu = synth.cu_seqlens_of([300, 77])
    plan = tm.tilemix_build_plan(cu, 6, 2, 64)
    T, hq, hkv, d = 377, 6, 2, 64
    _, tq, tk = tm.tilemix_query_sizes(cu)
    f16 = lambda *s: torch.zeros(*s, dtype=torch.float16)
    i8 = lambda *s: torch.zeros(*s, dtype=torch.int8)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
    plan_d = torch.from_numpy(plan)
    words = torch.zeros(hkv * tq, dtype=torch.int64)
    good = dict(q=f16(T, hq, d), k=f16(T, hkv, d), v=f16(T, hkv, d), k_i8=i8(T, hkv, d), k_scale=f32(hkv, tk),
                out=f16(T, hq, d))

    def call(**over):
        a = dict(good, **over)
        tm.tilemix_prefill_varlen_qinline(plan, plan_d, a["q"], a["k"], a["v"], a["k_i8"], a["k_scale"],
                                          words, a["out"])

    for name, bad in (("q", f16(T - 1, hq, d)), ("k", f16(T, hkv - 1, d)), ("v", f16(T, hkv, d - 8)),
                      ("k_i8", i8(T, hkv, d - 1)), ("k_scale", f32(hkv, tk - 1)), ("out", f16(T, hq - 1, d))):
        with pytest.raises(tm.TileMixError, match=name + " holds"):
            call(**{name: bad})
    with pytest.raises(tm.TileMixError, match="device tensor"):   # right sizes: next the device check
        call()
    with pytest.raises(tm.TileMixError, match="plan_d"):
        tm.tilemix_quantize_k(plan, plan_d[:-1], good["k"], good["k_i8"], good["k_scale"])
    with pytest.raises(tm.TileMixError, match="q holds"):          # decode queries are [B, Hq, d]
        tm.tilemix_decode_varlen(plan, plan_d, f16(1, hq, d), good["k_i8"], good["k_i8"], good["k_scale"],
                                 good["k_scale"], words, torch.zeros(16, dtype=torch.uint8), f16(2, hq, d))


def test_plan_checksum_refuses_a_modified_host_plan():
    cu = synth.cu_seqlens_of([4096] * 2)
    plan = tm.tilemix_build_plan(cu, 6, 2, 128)
    assert plan[14] != 0
    bad = plan.copy()
    bad[-1] ^= 1                      # one work unit's row changed
    fake = ctypes.c_void_p(1 << 20)
    rc = tm.lib().tilemix_quantize_k(bad.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, fake, None)
    assert rc == -1 and "checksum" in tm.tilemix_last_error()
    bad = plan.copy()
    bad[9] -= 1                       # work-unit count no longer matches the body
    rc = tm.lib().tilemix_quantize_k(bad.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, fake, None)
    assert rc == -1


def test_select_routing_adaptive_validation_and_counts():
    """The device word selection's argument checks (no launch) and its
    host-side counts, which equal the oracle's N8 and N_legal."""
    lens = [300, 0, 129, 4160]
    cu = synth.cu_seqlens_of(lens)
    plan = tm.tilemix_build_plan(cu, 2, 2, 64)
    lib = tm.lib()
    lib.tilemix_select_routing_adaptive.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_void_p]
    p = ctypes.c_void_p(plan.ctypes.data)
    fake = ctypes.c_void_p(16)
    assert lib.tilemix_select_routing_adaptive(p, fake, fake, 10001, fake, None, None, None) == -1
    assert "coverage_bp" in tm.tilemix_last_error()
    assert lib.tilemix_select_routing_adaptive(p, fake, fake, 5000, None, None, None, None) == -1
    assert "words_d" in tm.tilemix_last_error()
    assert lib.tilemix_select_routing_adaptive(p, fake, ctypes.c_void_p(20), 5000, fake, None, None, None) == -1
    assert "aligned" in tm.tilemix_last_error()
    # an empty batch: counts only, nothing launched
    empty = tm.tilemix_build_plan(synth.cu_seqlens_of([0, 0]), 2, 2, 64)
    n8 = np.full(2, -1, dtype=np.int64)
    nl = np.full(2, -1, dtype=np.int64)
    assert lib.tilemix_select_routing_adaptive(ctypes.c_void_p(empty.ctypes.data), fake, None, 5000, None,
                                               ctypes.c_void_p(n8.ctypes.data),
                                               ctypes.c_void_p(nl.ctypes.data), None) == 0
    assert list(n8) == [0, 0] and list(nl) == [0, 0]
    for cov in (0, 1, 2500, 7777, 10000):
        _, _, on8, onl = oracle.routing_words(lens, 2, "band", cov, 0)
        n8 = np.zeros(len(lens), dtype=np.int64)
        nl = np.zeros(len(lens), dtype=np.int64)
        # counts are filled before the pointer checks (words_d NULL: refused)
        assert lib.tilemix_select_routing_adaptive(p, fake, fake, cov, None, ctypes.c_void_p(n8.ctypes.data),
                                                   ctypes.c_void_p(nl.ctypes.data), None) == -1
        assert list(nl) == list(onl) and list(n8) == list(on8)
