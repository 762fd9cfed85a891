"""The allocation-free decode entry point (tilemix_decode_varlen_noalloc)
against the workspace one (tilemix_decode_varlen), through the C ABI: the
same kernels, so the fp16 outputs must be bit-identical, over two calls in a
row on one GPU (the second on a smaller batch, so it reuses the first call's
scratch); and against the CPU oracle within the decode bar."""

import numpy as np
import pytest

import oracle
import synth
import mixed_precision_attention_amd as tm

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _step_both(lens, hq, hkv, d, template, cov, seed):
    print(f"no-alloc decode lens={lens} hq={hq} hkv={hkv} d={d} {template} {cov}", flush=True)
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=seed)
    q_new = synth.decode_queries(q, cu)
    td = tm.TileMixDecode(cu, hq, hkv, d, template, cov, device="cuda")
    td.fill_cache(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    qd = torch.from_numpy(q_new).cuda()
    ref = torch.full((len(lens), hq, d), float("nan"), dtype=torch.float16, device="cuda")
    got = torch.full_like(ref, float("nan"))
    td.step(qd, ref)
    td.step(qd, got, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "no-alloc output differs"
    k_i8, ks, v_i8, vs = oracle.quantize_kv_cache(k, v, cu)
    want = oracle.decode_attention(q_new, k_i8, ks, v_i8, vs, td.words, cu, hq, hkv)
    err = np.abs(got.cpu().numpy().astype(np.float64) - want)
    assert err.max() <= 4e-3 and err.mean() <= 5e-4, (err.max(), err.mean())


def test_noalloc_two_calls_second_smaller():
    # first call: 3B shape at 2x4160 keys (g = 2) -- 0.27 MB of records
    _step_both([4160, 3000], 24, 8, 128, "sptrans", 7500, seed=5)
    # second call on the same GPU: fewer, shorter sequences, another head
    # count and d = 64 (every record it reads is written by this call)
    _step_both([300, 77, 0, 129, 1, 64], 4, 2, 64, "rowrandom", 5000, seed=6)


def test_noalloc_rejects_oversized_step():
    # B * Hq * ceil(max L / 256) * (d + 2) * 4 bytes > 32 MiB: refused on the
    # host, before any launch (the workspace form still takes it)
    lens = [65600, 1, 1, 1]
    plan_h = tm.tilemix_build_plan(synth.cu_seqlens_of(lens), 64, 8, 128)
    assert tm.tilemix_decode_workspace_size(plan_h) > 32 * 1024 * 1024
    T, (_, tq, tk) = int(synth.cu_seqlens_of(lens)[-1]), tm.tilemix_query_sizes(synth.cu_seqlens_of(lens))
    q = torch.zeros((len(lens), 64, 128), dtype=torch.float16, device="cuda")
    i8 = torch.zeros((T, 8, 128), dtype=torch.int8, device="cuda")
    f32 = torch.zeros((8, tk), dtype=torch.float32, device="cuda")
    words = torch.zeros((8, tq), dtype=torch.int64, device="cuda")
    plan_d = torch.from_numpy(plan_h).cuda()
    with pytest.raises(tm.TileMixError, match="scratch"):
        tm.tilemix_decode_varlen_noalloc(plan_h, plan_d, q, i8, i8, f32, f32, words, torch.empty_like(q))
