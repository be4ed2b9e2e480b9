"""K-cache writer on the GPU: the bytes it writes (codes and scales, every
layout, fp32 and bf16 input) equal the oracle's cache image exactly, skipped
rows and untouched bytes keep their canaries, and a cache written by it scores
like one written by the input generator."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ensure_built, log
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _keys(rng, N):
    k = rng.standard_normal((N, 128)).astype(np.float32)
    k *= rng.uniform(1e-4, 80, (N, 1)).astype(np.float32)
    k[0] = 0.0                                     # all-zero row
    k[1, :] = 0.0
    k[1, 7] = -3.0                                 # one value, negative
    k[2, ::2] = -0.0                               # signed zeros
    k[3, 0] = 1e30                                 # outlier: the rest underflows
    k[4] = np.float32(2.0 ** -130) * (1 + np.arange(128))   # subnormal inputs
    k[5, :32] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9] * 4  # E2M1 ties
    return k


def _run(dtype, layout, k_bf16, N=1000, P=64, pages=24, seed=0):
    rng = np.random.default_rng(seed)
    row_stride = 144 if layout == "row_inline" else None
    cache = synth._alloc_cache(dtype, pages, P, 128, row_stride, layout, True)
    k32 = _keys(rng, N)
    if k_bf16:
        kt = torch.from_numpy(k32).to(torch.bfloat16)
        k32 = kt.to(torch.float32).numpy()         # the exact values the kernel reads
        kdev = kt.cuda()
    else:
        kdev = torch.from_numpy(k32).cuda()
    slots = rng.permutation(pages * P)[:N].astype(np.int64)
    slots[rng.integers(0, N, 25)] = -1             # padding rows
    slots[rng.integers(0, N, 10)] = pages * P + 7  # past the pool
    data_dev = torch.from_numpy(cache.data.copy()).cuda()
    if cache.scale_offset >= 0:
        scale_ptr = data_dev.data_ptr() + cache.scale_offset
        scale_dev = None
    else:
        scale_dev = torch.from_numpy(cache.scale.copy()).cuda()
        scale_ptr = scale_dev.data_ptr()
    kv = idx.make_kv_cache(dtype, P, pages, data_dev, cache.page_stride, cache.row_stride,
                           scale_ptr, cache.scale_page_stride, cache.scale_row_stride)
    sm_dev = torch.from_numpy(slots).cuda()
    idx.idx_kv_cache_write(kdev, idx.IDX_KIN_BF16 if k_bf16 else idx.IDX_KIN_F32, 128, N, sm_dev,
                           kv)
    torch.cuda.synchronize()
    # oracle on a host copy of the same initial image
    ref = oracle.Cache(dtype, cache.data, cache.page_stride, cache.row_stride, cache.scale,
                       cache.scale_page_stride, cache.scale_row_stride, P, pages)
    oracle.kv_write(dtype, k32, slots, ref)
    got_data = data_dev.cpu().numpy()
    got_scale = None if scale_dev is None else scale_dev.cpu().numpy()
    return cache, got_data, got_scale


@pytest.mark.parametrize("dtype", [synth.FP8, synth.MXFP4])
@pytest.mark.parametrize("layout", ["separate", "page_block", "row_inline"])
@pytest.mark.parametrize("k_bf16", [False, True])
def test_kv_write_matches_oracle_bytes(dtype, layout, k_bf16):
    log("kv write dtype %d layout %s bf16 %d" % (dtype, layout, k_bf16))
    cache, got_data, got_scale = _run(dtype, layout, k_bf16)
    assert np.array_equal(got_data, cache.data), "data bytes differ from the oracle"
    if got_scale is not None:
        assert np.array_equal(got_scale, cache.scale), "scale bytes differ from the oracle"


def test_kv_write_large_and_ragged():
    """Full-width batch: every slot of a 1024-page pool of 64-row pages (65536
    rows, a ragged multiple of the 4-row work group minus one), FP8."""
    log("kv write large")
    P, pages, N = 64, 1024, 65535
    rng = np.random.default_rng(11)
    cache = synth._alloc_cache(synth.FP8, pages, P, 128, None, "separate", True)
    k32 = (rng.standard_normal((N, 128)) * 2).astype(np.float32)
    slots = rng.permutation(pages * P)[:N].astype(np.int64)
    data_dev = torch.from_numpy(cache.data.copy()).cuda()
    scale_dev = torch.from_numpy(cache.scale.copy()).cuda()
    kv = idx.make_kv_cache(synth.FP8, P, pages, data_dev, cache.page_stride, cache.row_stride,
                           scale_dev, cache.scale_page_stride, cache.scale_row_stride)
    idx.idx_kv_cache_write(torch.from_numpy(k32).cuda(), idx.IDX_KIN_F32, 128, N,
                           torch.from_numpy(slots).cuda(), kv)
    torch.cuda.synchronize()
    ref = oracle.Cache(synth.FP8, cache.data, cache.page_stride, cache.row_stride, cache.scale,
                       cache.scale_page_stride, cache.scale_row_stride, P, pages)
    oracle.kv_write(synth.FP8, k32, slots, ref)
    assert np.array_equal(data_dev.cpu().numpy(), cache.data)
    assert np.array_equal(scale_dev.cpu().numpy(), cache.scale)


def test_written_cache_scores_like_the_generated_one():
    """Keys written by the writer into a decode case's pages give the same
    logits, bit for bit, as the generator's own quantized keys."""
    log("kv write then score")
    case = synth.decode_case([700, 1500], next_n=1, P=64, k=64, W=1536, seed=12, canary=False)
    from gpu_util import DeviceCase, run_decode
    dc = DeviceCase(case)
    logits_ref, _, _ = run_decode(dc)
    # regenerate the same keys: decode_case draws them from its seeded stream
    rng = synth.rng_for(12)
    npg = (case.lens + 63) // 64
    _ = rng.permutation(case.cache.num_pages)
    keys, slots = [], []
    for b in range(case.B):
        L = int(case.lens[b])
        kb = rng.standard_normal((L, 128), dtype=np.float32)
        keys.append(kb)
        pages = case.block_tables[b, :npg[b]].astype(np.int64)
        rows = (pages[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)[:L]
        slots.append(rows)
    k = np.concatenate(keys)
    sl = np.concatenate(slots)
    dc.t["kdata"].fill_(0x7F)
    if dc.t["kscale"] is not None:
        dc.t["kscale"].fill_(0)
    idx.idx_kv_cache_write(torch.from_numpy(k).cuda(), idx.IDX_KIN_F32, 128, k.shape[0],
                           torch.from_numpy(sl).cuda(), dc.kv)
    logits_new, _, _ = run_decode(dc)
    E = case.lens
    for b in range(case.B):
        assert torch.equal(logits_new[b, :E[b]], logits_ref[b, :E[b]])
