"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances: bf16 outputs max |gpu - oracle| <= 2e-2; fp32 GEMM outputs
componentwise |gpu - oracle| <= 1e-3 * sum_k |a_k w_k|; integer and copy
work bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import deterministic_paged_attention_amd as bi
import oracle
import synth
from harness import (DEV, PagedKV, Request, first_mismatch, logical_k, logical_v, nan_cache, oracle_rows,
                     page_table_tensor,
                     run_step)

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def _max_err(gpu_rows, ref_rows):
    return max(float(np.max(np.abs(synth.to_f64(gpu_rows[k]) - ref_rows[k]))) for k in ref_rows)


# ---------------------------------------------------------------- a1: slot mapping + KV write

def test_slot_mapping_and_kv_write_bit_exact():
    torch.manual_seed(0)
    cfg = bi.AttnConfig(4, 2, 64)
    geom = synth.Geometry(4, 2, 64, 16)
    lengths, q_lens = [17, 33, 64, 100], [17, 5, 1, 37]
    plan = synth.random_page_plan(lengths, 16, seed=3, slack=5)
    pt_host = plan.table(stride=9).numpy()
    pt_host[2, 6] = 999  # an entry beyond the 4 pages sequence 2 uses: never read
    pt = torch.tensor(pt_host, device=DEV)
    sl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    qsl_h = np.concatenate([[0], np.cumsum(q_lens)])
    qsl = torch.tensor(qsl_h, dtype=torch.int32, device=DEV)
    T = int(qsl_h[-1])
    slots = bi.bi_slot_mapping(pt, sl, qsl, T, 16, plan.num_pages).cpu().numpy()
    ref = oracle.slot_mapping_ref(pt_host, lengths, qsl_h, 16)
    assert slots.tolist() == ref.tolist()

    kn = torch.cat([synth.token_kv(geom, 50 + s, L)[0][L - q_lens[s]:] for s, L in enumerate(lengths)])
    vn = torch.cat([synth.token_kv(geom, 50 + s, L)[1][L - q_lens[s]:] for s, L in enumerate(lengths)])
    kc = nan_cache(cfg.k_cache_shape(plan.num_pages))
    vc = nan_cache(cfg.v_cache_shape(plan.num_pages))
    bi.bi_kv_write(cfg, kn.to(DEV), vn.to(DEV), torch.tensor(slots, device=DEV), kc, vc)
    k0 = np.full((plan.num_pages, 16, 2, 64), np.nan)
    v0 = k0.copy()
    kr, vr = oracle.kv_write_ref(k0, v0, synth.to_f64(kn), synth.to_f64(vn), ref, 16)
    np.testing.assert_array_equal(logical_k(kc), kr)   # NaN == NaN positionally
    np.testing.assert_array_equal(logical_v(vc), vr)
    # the same write with the slots computed in the write kernel from the page table
    kc2 = nan_cache(cfg.k_cache_shape(plan.num_pages))
    vc2 = nan_cache(cfg.v_cache_shape(plan.num_pages))
    bi.bi_kv_write_paged(cfg, kn.to(DEV), vn.to(DEV), pt, sl, qsl, kc2, vc2)
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))


@pytest.mark.parametrize("Hq,Hk,D", [(32, 8, 128), (8, 4, 256)])
def test_kv_write_paged_is_slot_mapping_then_kv_write(Hq, Hk, D):
    """Out-of-pool and negative entries (skipped tokens), ragged q_len, strided k/v rows."""
    cfg = bi.AttnConfig(Hq, Hk, D)
    lengths, q_lens = [40, 7, 300, 16], [3, 7, 1, 16]
    num_pages = 30
    pt_host = np.full((4, 20), -1, dtype=np.int32)
    pt_host[0, :3] = [4, 29, 31]          # 31 is past the pool: its tokens are skipped
    pt_host[1, :1] = [0]
    pt_host[2, :19] = np.arange(5, 24)
    pt_host[3, :1] = [-7]                 # negative entry: skipped
    pt = torch.tensor(pt_host, device=DEV)
    sl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    qsl_h = np.concatenate([[0], np.cumsum(q_lens)])
    qsl = torch.tensor(qsl_h, dtype=torch.int32, device=DEV)
    T = int(qsl_h[-1])
    rows = synth.normal_bf16((T, 2 * Hk * D + 16), 620).to(DEV)
    kn = rows[:, : Hk * D].view(T, Hk, D)
    vn = rows[:, Hk * D + 16:].view(T, Hk, D)
    outs = []
    for paged in (False, True):
        kc = nan_cache(cfg.k_cache_shape(num_pages))
        vc = nan_cache(cfg.v_cache_shape(num_pages))
        if paged:
            bi.bi_kv_write_paged(cfg, kn, vn, pt, sl, qsl, kc, vc)
        else:
            slots = bi.bi_slot_mapping(pt, sl, qsl, T, 16, num_pages)
            bi.bi_kv_write(cfg, kn, vn, slots, kc, vc)
        outs.append((kc, vc))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_slot_mapping_out_of_range_pages_give_minus_one():
    pt = torch.tensor([[0, 7, -3]], dtype=torch.int32, device=DEV)
    sl = torch.tensor([40], dtype=torch.int32, device=DEV)
    qsl = torch.tensor([0, 40], dtype=torch.int32, device=DEV)
    slots = bi.bi_slot_mapping(pt, sl, qsl, 40, 16, 5).cpu().numpy()
    assert slots[:16].tolist() == list(range(16))
    assert (slots[16:] == -1).all()


# ---------------------------------------------------------------- a2 + a3: attention parity

def _decode_case(geom, cfg, lengths, seed, order=None, stride_extra=0):
    reqs = {i: Request(seed * 100 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, sum(synth.pages_needed(L, 16) for L in lengths) + 7, seed)
    order = list(range(len(lengths))) if order is None else order
    run_step(kv, reqs, [(i, lengths[i] - 1) for i in order], attention=False)
    out = run_step(kv, reqs, [(i, 1) for i in order], stride_extra=stride_extra)
    return reqs, out


@pytest.mark.parametrize("S", [32, 256])
def test_config1_tiny_decode_parity(S):
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=S)
    lengths = [17, 33, 64, 100]
    reqs, out = _decode_case(geom, cfg, lengths, seed=1, order=[2, 0, 3, 1])
    ref = oracle_rows(reqs, list(out.keys()), geom, 0)
    assert _max_err(out, ref) <= BF16_TOL


@pytest.mark.parametrize("window", [0, 100])
def test_prefill_chunks_parity_llama_shape(window):
    geom = synth.Geometry(32, 8, 128, 16)
    cfg = bi.AttnConfig(32, 8, 128, split_size=256, window=window)
    lengths = [300, 777, 1029]
    reqs = {i: Request(900 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 200, seed=9)
    run_step(kv, reqs, [(0, 250), (1, 700), (2, 900)], attention=False)
    out = run_step(kv, reqs, [(0, 50), (1, 77), (2, 129)])
    keys = [k for k in out if k[1] % 7 == 0 or k[1] == lengths[k[0]] - 1]
    ref = oracle_rows(reqs, keys, geom, window)
    assert _max_err(out, ref) <= BF16_TOL


def test_gemma_shape_d256_window_parity():
    geom = synth.Geometry(8, 4, 256, 16)
    cfg = bi.AttnConfig(8, 4, 256, split_size=256, window=1024)
    lengths = [1500, 2100, 40]
    reqs = {i: Request(700 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 260, seed=4)
    run_step(kv, reqs, [(0, 1499), (1, 2030), (2, 10)], attention=False)
    out = run_step(kv, reqs, [(0, 1), (1, 70), (2, 30)])
    keys = [k for k in out if k[1] % 5 == 0 or k[1] == lengths[k[0]] - 1]
    ref = oracle_rows(reqs, keys, geom, 1024)
    assert _max_err(out, ref) <= BF16_TOL


def test_single_key_is_v0_bitwise():
    geom = synth.Geometry(32, 8, 128, 16)
    cfg = bi.AttnConfig(32, 8, 128)
    reqs = {0: Request(5, 1, geom), 1: Request(6, 1, geom)}
    kv = PagedKV(cfg, 8, seed=2)
    out = run_step(kv, reqs, [(0, 1), (1, 1)])
    for rid in (0, 1):
        v0 = reqs[rid].v[0]                         # [H_kv, D] bf16
        expect = v0.repeat_interleave(4, dim=0)     # head h reads KV head h // 4
        assert torch.equal(out[(rid, 0)].view(torch.int16), expect.view(torch.int16))


@pytest.mark.parametrize("Hq,Hk,D", [(32, 8, 128), (8, 4, 256), (4, 2, 64)])
def test_window_of_one_returns_own_value_bitwise(Hq, Hk, D):
    """With a window of one key every row sees only its own position: one
    score, weight exp(0) = 1, sum 1, so the output must be bf16(v_p) of the
    row's KV head, bitwise, for prefill chunks and decode rows alike, at
    positions deep inside long contexts (many splits before the window)."""
    geom = synth.Geometry(Hq, Hk, D, 16)
    cfg = bi.AttnConfig(Hq, Hk, D, split_size=256, window=1)
    lengths = [700, 1300, 45]
    reqs = {i: Request(820 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 180, seed=12)
    run_step(kv, reqs, [(0, 600), (1, 1200), (2, 5)], attention=False)
    out = run_step(kv, reqs, [(0, 99), (1, 37), (2, 39)])
    out.update(run_step(kv, reqs, [(0, 1), (1, 1), (2, 1)]))
    G = Hq // Hk
    for (rid, p), row in out.items():
        expect = reqs[rid].v[p].repeat_interleave(G, dim=0)
        assert torch.equal(row.view(torch.int16), expect.view(torch.int16)), (rid, p)


def test_gemma_shape_32k_context_decode_parity():
    """The longest context of the decoder workload: a global (no window) layer
    of the Gemma-shaped geometry decoding at position 32767 (128 splits per
    row merged), next to a short sequence in the same batch."""
    geom = synth.Geometry(8, 4, 256, 16)
    cfg = bi.AttnConfig(8, 4, 256, split_size=256)
    lengths = [32768, 300]
    reqs = {i: Request(960 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 2100, seed=13)
    run_step(kv, reqs, [(0, 32767), (1, 299)], attention=False)
    out = run_step(kv, reqs, [(0, 1), (1, 1)])
    ref = oracle_rows(reqs, list(out.keys()), geom, 0)
    assert _max_err(out, ref) <= BF16_TOL


def test_split_phase_partials_parity():
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=32)
    lengths, q_lens = [100, 70], [3, 20]
    reqs = {i: Request(40 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 20, seed=8)
    run_step(kv, reqs, [(0, lengths[0]), (1, lengths[1])], attention=False)
    tabs = [kv.tables[0], kv.tables[1]]
    pt = page_table_tensor(tabs, 8).to(DEV)
    sl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    qsl_h = np.array([0, 3, 23])
    qsl = torch.tensor(qsl_h, dtype=torch.int32, device=DEV)
    q = torch.cat([reqs[0].q[97:100], reqs[1].q[50:70]]).to(DEV)
    ws = bi.alloc_workspace(bi.bi_paged_attention_workspace_size(cfg, 2, 23, 100))
    bi.bi_paged_attention_split(cfg, q, kv.k, kv.v, pt, sl, qsl, 100, ws)
    ns = 4
    ml, acc = bi.workspace_views(cfg, ws, 23, ns)
    ml, acc = ml.cpu().double().numpy(), acc.cpu().double().numpy()
    kc, vc = logical_k(kv.k), logical_v(kv.v)
    pt_h = page_table_tensor(tabs, 8).numpy()
    m, l, a, valid = oracle.split_partials_ref(synth.to_f64(q.cpu()), kc, vc, pt_h, lengths, qsl_h, 2, 16, 32)
    R = 23 * 4
    valid = valid.reshape(R, ns)
    gm, gl, ga = ml[:, :, 0][valid], ml[:, :, 1][valid], acc[valid]
    om, ol, oa = m.reshape(R, ns)[valid], l.reshape(R, ns)[valid], a.reshape(R, ns, 64)[valid]
    assert np.max(np.abs(gm - om)) <= 1e-3 * max(1.0, np.max(np.abs(om)))
    assert np.max(np.abs(gl / ol - 1)) <= 1e-2
    assert np.max(np.abs(ga / gl[:, None] - oa / ol[:, None])) <= BF16_TOL


def test_merge_phase_parity_on_synthetic_partials():
    cfg = bi.AttnConfig(4, 2, 64, split_size=32)
    T, H, D, L = 5, 4, 64, 130          # one sequence of 130 keys, 5 query rows -> 5 splits
    ns = 5
    rng = torch.Generator().manual_seed(77)
    m = (torch.rand((T * H, ns), generator=rng) * 20 - 10).double()
    l = (torch.rand((T * H, ns), generator=rng) * 30 + 1).double()
    a = torch.randn((T * H, ns, D), generator=rng).double() * l[:, :, None]
    ws = bi.alloc_workspace(bi.bi_paged_attention_workspace_size(cfg, 1, T, L))
    ml, acc = bi.workspace_views(cfg, ws, T, ns)
    ml[:, :, 0] = m.float().to(DEV)
    ml[:, :, 1] = l.float().to(DEV)
    acc[:] = a.to(torch.bfloat16).to(DEV)  # the workspace keeps each split's accumulator in bf16
    sl = torch.tensor([L], dtype=torch.int32, device=DEV)
    qsl = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    out = bi.bi_paged_attention_merge(cfg, sl, qsl, T, L, ws).cpu()
    mf, lf = (x.float().double().numpy() for x in (m, l))
    af = a.to(torch.bfloat16).double().numpy()
    # row t sits at p = L - T + t and reads the splits 0 .. p // 32 only
    valid = np.zeros((T, H, ns), dtype=bool)
    for t in range(T):
        valid[t, :, : (L - T + t) // 32 + 1] = True
    ref = oracle.merge_ref(mf.reshape(T, H, ns), lf.reshape(T, H, ns), af.reshape(T, H, ns, D), valid)
    assert np.max(np.abs(synth.to_f64(out) - ref)) <= BF16_TOL


def test_full_size_llama_decode_sampled_parity():
    """8B-shaped decode at B = 256 (the benchmarked launch), oracle on sampled sequences."""
    from synth.workloads import build_decode_workload
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    wl = build_decode_workload(32, 8, 128, batch=256, seed=2000)
    out = bi.bi_paged_attention(cfg, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                wl.max_seq_len)
    torch.cuda.synchronize()
    sample = [0, 17, 101, 255]
    errs = []
    for s in sample:
        kk, vv, table, L = wl.host_sequence(s)
        q = synth.to_f64(wl.q[s:s + 1].cpu())
        ref = oracle.attention_ref(q, kk, vv, table, [L], [0, 1], 8, 16)
        errs.append(float(np.max(np.abs(synth.to_f64(out[s:s + 1].cpu()) - ref))))
    assert max(errs) <= BF16_TOL, errs


# ---------------------------------------------------------------- a4: RMSNorm

@pytest.mark.parametrize("M,H", [(1, 4096), (7, 4096), (64, 4096), (3, 12288)])
def test_rmsnorm_parity(M, H):
    x = synth.normal_bf16((M, H), 401)
    g = synth.normal_bf16((H,), 402, std=0.1, mean=1.0)
    y = bi.bi_rmsnorm(x.to(DEV), g.to(DEV), 1e-5).cpu()
    ref = oracle.rmsnorm_ref(synth.to_f64(x), synth.to_f64(g), 1e-5)
    assert np.max(np.abs(synth.to_f64(y) - ref)) <= BF16_TOL


def test_rmsnorm_ragged_hidden_and_strides():
    H = 2568                              # not a multiple of the 2048-element sweep of a workgroup
    x = synth.normal_bf16((9, H + 8), 403)
    g = synth.normal_bf16((H,), 404, std=0.1, mean=1.0)
    xd = x.to(DEV)[:, :H]
    out = torch.zeros((9, H + 16), dtype=torch.bfloat16, device=DEV)
    bi.bi_rmsnorm(xd, g.to(DEV), 1e-6, out=out[:, :H])
    ref = oracle.rmsnorm_ref(synth.to_f64(x[:, :H]), synth.to_f64(g), 1e-6)
    assert np.max(np.abs(synth.to_f64(out[:, :H].cpu()) - ref)) <= BF16_TOL
    assert (out[:, H:].float() == 0).all()


@pytest.mark.parametrize("M,F,K", [(1, 10240, 2560), (4, 10240, 2560), (16, 10240, 2560), (7, 4096, 1024),
                                   (3, 100, 96), (16, 24, 4128), (4, 6144, 2048), (5, 14336, 4096)])
def test_gemm_gated_gelu_is_gemm_then_gated_gelu(M, F, K):
    """The gated skinny product (gate and up rows of a [gate | up] weight in one
    workgroup, the activation in its epilogue) against bi_gemm + bi_gated_gelu,
    bitwise, with wide-ranging inputs (the activation's tanh saturates), ragged
    F and a K tail; and against the oracle's gated GELU of the GEMM."""
    g = torch.Generator(device=DEV)
    g.manual_seed(M * 131 + F + K)
    a = (torch.randn(M, K, device=DEV, generator=g) * 2.0).to(torch.bfloat16)
    w = (torch.randn(2 * F, K, device=DEV, generator=g) * 0.05).to(torch.bfloat16)
    fused = bi.bi_gemm_gated_gelu(a, w)
    gu = bi.bi_gemm(a, w)
    ref = bi.bi_gated_gelu(gu)
    assert first_mismatch(fused, ref) is None
    # strided rows of a and out
    a2 = torch.zeros(M, K + 40, dtype=torch.bfloat16, device=DEV)
    a2[:, :K] = a
    out2 = torch.full((M, F + 24), 7.0, dtype=torch.bfloat16, device=DEV)
    bi.bi_gemm_gated_gelu(a2[:, :K], w, out=out2[:, :F])
    assert first_mismatch(out2[:, :F], ref) is None
    assert bool((out2[:, F:].float() == 7.0).all())
    # oracle: gated GELU of the bf16 products (the GEMM's own rounding taken as given)
    gu64 = synth.to_f64(gu.cpu())
    want = oracle.gated_gelu_ref(gu64)
    a_abs = np.abs(want)
    tol = np.where(a_abs < 8.0, 2e-2, np.ldexp(1.0, np.frexp(a_abs)[1] - 8))   # 2e-2, one bf16 spacing from 8 on
    assert bool(np.all(np.abs(synth.to_f64(fused.cpu()) - want) <= tol))


@pytest.mark.parametrize("M,H", [(1, 2560), (7, 4096), (256, 2560), (3, 8), (5, 8200), (2, 16384)])
def test_add_rmsnorm_is_add_then_rmsnorm(M, H):
    """The fused residual add + norm equals the two separate launches bit for
    bit, and both equal the oracle's norm of the bf16-rounded sum."""
    a = synth.normal_bf16((M, H), 405).to(DEV)
    b = synth.normal_bf16((M, H), 406, std=3.0).to(DEV)
    g = synth.normal_bf16((H,), 407, std=0.1, mean=1.0).to(DEV)
    s_ref = bi.bi_add(a, b)
    y_ref = bi.bi_rmsnorm(s_ref, g, 1e-6)
    s, y = bi.bi_add_rmsnorm(a, b, g, 1e-6)
    assert torch.equal(s.view(torch.int16), s_ref.view(torch.int16))
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    sum64 = synth.to_f64(a.cpu()) + synth.to_f64(b.cpu())
    # the fp64 sum of two bf16 values is exact: rounded to fp32, then to bf16
    assert np.array_equal(synth.to_f64(s.cpu()),
                          synth.to_f64(torch.from_numpy(sum64).to(torch.float32).to(torch.bfloat16)))
    ref = oracle.rmsnorm_ref(synth.to_f64(s.cpu()), synth.to_f64(g.cpu()), 1e-6)
    assert np.max(np.abs(synth.to_f64(y.cpu()) - ref)) <= BF16_TOL
    # in place on a, with strided rows
    big = torch.zeros((M, H + 24), dtype=torch.bfloat16, device=DEV)
    big[:, :H] = a
    out = torch.zeros((M, H + 8), dtype=torch.bfloat16, device=DEV)
    bi.bi_add_rmsnorm(big[:, :H], b, g, 1e-6, sum_out=big[:, :H], out=out[:, :H])
    assert torch.equal(big[:, :H].view(torch.int16), s_ref.view(torch.int16))
    assert torch.equal(out[:, :H].view(torch.int16), y_ref.view(torch.int16))
    assert (big[:, H:].float() == 0).all() and (out[:, H:].float() == 0).all()


# ---------------------------------------------------------------- a5: GEMM

@pytest.mark.parametrize("M,N,K", [(37, 300, 4096), (16, 300, 4128), (64, 20000, 2080), (200, 5000, 96),
                                   (129, 12000, 2080), (100, 70000, 1056), (200, 20480, 2080), (240, 2560, 2080),
                                   (300, 9000, 4128), (400, 16400, 1056), (1024, 16400, 1056)])
def test_gemm_small_integers_exact_fp32(M, N, K):
    """Integer inputs make every correct fp32-accumulating product exact, so any
    lost, repeated or misplaced K step shows.  The shapes reach the skinny kernel
    and each ring-tile bracket of M and N, with K both a multiple of every slice
    width and ragged (a partly filled last slice, or a single short one)."""
    a = synth.small_int_bf16((M, K), 501)
    w = synth.small_int_bf16((N, K), 502)
    c = bi.bi_gemm(a.to(DEV), w.to(DEV), out_dtype=torch.float32).cpu()
    ref = oracle.gemm_ref(synth.to_f64(a), synth.to_f64(w))
    assert np.array_equal(c.double().numpy(), ref)


@pytest.mark.parametrize("M,N", [(1, 14336), (7, 1000), (64, 2048), (300, 777)])
def test_gemm_parity(M, N):
    a = synth.normal_bf16((M, 4096), 511)
    w = synth.normal_bf16((N, 4096), 512, std=0.02)
    ad, wd = a.to(DEV), w.to(DEV)
    c32 = bi.bi_gemm(ad, wd, out_dtype=torch.float32).cpu().double().numpy()
    c16 = synth.to_f64(bi.bi_gemm(ad, wd).cpu())
    ref = oracle.gemm_ref(synth.to_f64(a), synth.to_f64(w))
    bound = oracle.gemm_abs_ref(synth.to_f64(a), synth.to_f64(w))
    assert np.all(np.abs(c32 - ref) <= 1e-3 * bound)
    assert np.max(np.abs(c16 - ref)) <= BF16_TOL


@pytest.mark.parametrize("M", [1, 33, 129, 300])
@pytest.mark.parametrize("K", [96, 4128])
def test_gemm_ragged_k_tails_and_strides(M, K):
    """K with an odd number of 32-wide steps (a half-empty last 64-wide slice),
    M and N off every tile size, and row strides larger than K."""
    N = 77
    a = synth.normal_bf16((M, K + 24), 531)
    w = synth.normal_bf16((N, K + 40), 532, std=0.02)
    ad, wd = a.to(DEV)[:, :K], w.to(DEV)[:, :K]
    out = torch.full((M, N + 5), 7.0, dtype=torch.float32, device=DEV)
    bi.bi_gemm(ad, wd, out=out[:, :N])
    ref = oracle.gemm_ref(synth.to_f64(a[:, :K]), synth.to_f64(w[:, :K]))
    bound = oracle.gemm_abs_ref(synth.to_f64(a[:, :K]), synth.to_f64(w[:, :K]))
    got = out.cpu().double().numpy()
    assert np.all(np.abs(got[:, :N] - ref) <= 1e-3 * bound)
    assert np.all(got[:, N:] == 7.0)


@pytest.mark.parametrize("N", [1000, 6144, 8192, 12288, 20000])
def test_gemm_tile_configurations_agree_bitwise(N):
    """The tile configuration follows M and N (every M bracket and N bracket is
    visited here); each row of c must equal, bit for bit, that row computed
    alone (M = 1), and agree with the oracle."""
    K = 2560
    a = synth.normal_bf16_device((300, K), 541)
    w = synth.normal_bf16_device((N, K), 542, std=0.02)
    single = {r: bi.bi_gemm(a[r:r + 1], w, out_dtype=torch.float32) for r in (0, 16, 32, 64, 128, 299)}
    for M in (16, 17, 33, 65, 100, 129, 257, 300):
        c = bi.bi_gemm(a[:M], w, out_dtype=torch.float32)
        for r, ref in single.items():
            if r < M:
                assert first_mismatch(c[r:r + 1], ref) is None, (M, r)
    rows = [0, 299]
    ah, wh = synth.to_f64(a[rows].cpu()), synth.to_f64(w[:64].cpu())
    got = torch.cat([single[r][:, :64] for r in rows]).cpu().double().numpy()
    assert np.all(np.abs(got - oracle.gemm_ref(ah, wh)) <= 1e-3 * oracle.gemm_abs_ref(ah, wh))


@pytest.mark.parametrize("N,K", [(100, 96), (1000, 4128), (2560, 2048), (2560, 10240), (4096, 2560),
                                 (6144, 4096), (8192, 2560)])
def test_gemm_skinny_rows_agree_with_tiles_bitwise(N, K):
    """M <= 16 products run the skinny kernel (16-row weight blocks, a's rows
    loaded by the computing wave), M = 17 output tiles.  Every row of the
    skinny product must equal, bit for bit, that row of the M = 17 product, in
    bf16 and fp32, also through row strides and a ragged last slice of K; and
    agree with the oracle."""
    a = synth.normal_bf16_device((17, K), 551 + K)
    w = synth.normal_bf16_device((N, K), 552 + N, std=0.02)
    for out_dtype in (torch.bfloat16, torch.float32):
        tiles = bi.bi_gemm(a, w, out_dtype=out_dtype)
        for M in (1, 3, 4, 16):
            c = bi.bi_gemm(a[:M], w, out_dtype=out_dtype)
            assert first_mismatch(c, tiles[:M]) is None, (M, out_dtype)
    # strided a and c: rows K + 40 apart, columns past N untouched
    a2 = torch.zeros(4, K + 40, dtype=torch.bfloat16, device=DEV)
    a2[:, :K] = a[:4]
    c2 = torch.full((4, N + 24), 7.0, dtype=torch.bfloat16, device=DEV)
    bi.bi_gemm(a2[:, :K], w, out=c2[:, :N])
    assert first_mismatch(c2[:, :N], bi.bi_gemm(a[:4], w)) is None
    assert bool((c2[:, N:].float() == 7.0).all())
    cols = sorted({0, 1, N // 3, N // 2 + 5, N - 1})
    ah, wh = synth.to_f64(a[:4].cpu()), synth.to_f64(w[cols].cpu())
    got = bi.bi_gemm(a[:4], w, out_dtype=torch.float32)[:, cols].cpu().double().numpy()
    assert np.all(np.abs(got - oracle.gemm_ref(ah, wh)) <= 1e-3 * oracle.gemm_abs_ref(ah, wh))


def test_gemm_lm_head_full_size_sampled():
    """M = 1024 x N = 128256 x K = 4096 with fp32 logits; oracle on sampled entries."""
    M, N, K = 1024, 128256, 4096
    a = synth.normal_bf16_device((M, K), 521)
    w = synth.normal_bf16_device((N, K), 522, std=0.02)
    c = bi.bi_gemm(a, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 511, 1023])
    cols = torch.tensor([0, 5, 77777, 128255, 64000, 12345])
    ah = synth.to_f64(a[rows].cpu())
    wh = synth.to_f64(w[cols].cpu())
    ref = oracle.gemm_ref(ah, wh)
    got = c[rows][:, cols].cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 1e-3 * oracle.gemm_abs_ref(ah, wh))


@pytest.mark.parametrize("nbytes", [0, 16, 4096 * 16 + 48, (64 << 20) + 1040])
def test_stream_read_reads_every_byte(nbytes):
    """The streaming-read reference (measurement only) must read the whole
    buffer: the xor of its sink equals the xor of the buffer's 32-bit words,
    and a one-word change anywhere (first, middle, last chunk) changes it."""
    words = nbytes // 4
    src = torch.randint(-2**31, 2**31 - 1, (words,), dtype=torch.int32, generator=torch.Generator().manual_seed(9))
    expect = int(np.bitwise_xor.reduce(src.numpy().view(np.uint32))) if words else 0
    d = src.to(DEV)
    got = int(np.bitwise_xor.reduce(bi.bi_bench_stream_read(d).cpu().numpy().view(np.uint32)))
    assert got == expect
    for pos in sorted({0, words // 2, words - 1}) if words else []:
        d2 = d.clone()
        d2[pos] ^= 0x5A5A5A5A
        flipped = int(np.bitwise_xor.reduce(bi.bi_bench_stream_read(d2).cpu().numpy().view(np.uint32)))
        assert flipped == expect ^ 0x5A5A5A5A


@pytest.mark.parametrize("rounds", [4, 64])
def test_mfma_peak_runs_every_instruction(rounds):
    """The MFMA throughput reference (measurement only): with all-one
    fragments each MFMA adds 32 to every accumulator element, so each wave's
    sink is 8 accumulators x 32 x rounds exactly, and the reported flop count
    is waves x rounds x 8 x 16384."""
    sink, flops = bi.bi_bench_mfma_peak(rounds, value=1.0)
    got = sink.cpu().numpy()
    assert np.all(got == 8.0 * 32.0 * rounds)
    assert flops == got.size * rounds * 8 * 16384
