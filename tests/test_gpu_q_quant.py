"""Query quantization with the weight fold on the GPU: codes, scales and
weights equal the oracle's bit for bit (FP8 folded and unfolded, MXFP4; fp32
and bf16 input; padded row strides; in-place weights), rows past R stay
untouched, and a query quantized here scores, through the paged scores and
top-k, like the oracle's quantized query."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DeviceCase, check_logits, check_topk_band, ensure_built, log,
                      oracle_decode_rows, run_decode)
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu

ROW = 64 * 128


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _rows(rng, R):
    x = rng.standard_normal((R, 64, 128)).astype(np.float32)
    x *= np.exp2(rng.integers(-8, 9, size=(R, 64, 1))).astype(np.float32)
    x[:, :, ::19] = 0.0
    x[0] = 0.0                                            # all-zero row
    x[1, 5:, :] = -0.0                                    # signed zeros
    x[2, 0, 0] = 3e37                                     # outlier: the rest underflows
    x[3] = np.float32(2.0 ** -135) * (1 + np.arange(128))  # subnormal inputs
    x[4, :, :32] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9] * 4  # E2M1 ties
    x[4, 7, :8] = [448.0, 224.0, 240.0, 232.0, 0.001953125, 0.0009765625, -0.0029296875, 1.0]
    return x


def _quantize(dtype, x32, x_dev, ld, w, c, fold, in_place=False, pad_rows=1):
    """Runs the library; returns (q, q_scale or None, weights) on the host and
    checks that the padding row after the R rows kept its canary."""
    R = x32.shape[0]
    qbytes = ROW if dtype == synth.FP8 else ROW // 2
    q = torch.full(((R + pad_rows) * qbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    if dtype == synth.FP8:
        qs = None if fold else torch.full((R + pad_rows,), -7.0, dtype=torch.float32,
                                          device="cuda")
    else:
        qs = torch.full(((R + pad_rows) * 256,), 0x5A, dtype=torch.uint8, device="cuda")
    w_dev = torch.from_numpy(w).cuda()
    wo = w_dev if in_place else torch.full((R + pad_rows, 64), -1.0, dtype=torch.float32,
                                           device="cuda")
    out = idx.make_query(dtype, q, qs, wo)
    idx.idx_quantize_query(x_dev, idx.IDX_KIN_BF16 if x_dev.dtype == torch.bfloat16
                           else idx.IDX_KIN_F32, ld, R, w_dev, c, out)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    assert np.all(qh[R * qbytes:] == 0xA5), "bytes past the last row were written"
    if qs is not None:
        qsh = qs.cpu().numpy()
        if dtype == synth.FP8:
            assert np.all(qsh[R:] == -7.0)
            qsh = qsh[:R]
        else:
            assert np.all(qsh[R * 256:] == 0x5A)
            qsh = qsh[:R * 256].reshape(R, 64, 4)
    else:
        qsh = None
    woh = wo.cpu().numpy()
    if not in_place:
        assert np.all(woh[R:] == -1.0)
    return qh[:R * qbytes].reshape(R, 64, -1), qsh, woh[:R]


@pytest.mark.parametrize("dtype,fold", [(synth.FP8, True), (synth.FP8, False),
                                        (synth.MXFP4, False)])
@pytest.mark.parametrize("x_bf16", [False, True])
@pytest.mark.parametrize("ld", [ROW, ROW + 24])
def test_quantize_query_matches_oracle_bytes(dtype, fold, x_bf16, ld):
    log("q quant dtype %d fold %d bf16 %d ld %d" % (dtype, fold, x_bf16, ld))
    rng = np.random.default_rng(100 + ld % 7 + 2 * x_bf16)
    R = 37
    x32 = _rows(rng, R)
    w = rng.standard_normal((R, 64)).astype(np.float32)
    w[6] = 0.0
    w[7, ::3] *= -1e-30
    c = 0.0883883
    buf = np.zeros((R, ld), dtype=np.float32)
    buf[:, :ROW] = x32.reshape(R, ROW)
    buf[:, ROW:] = np.nan                      # never read
    if x_bf16:
        xt = torch.from_numpy(buf).to(torch.bfloat16)
        x32 = xt.to(torch.float32).numpy()[:, :ROW].reshape(R, 64, 128)
        x_dev = xt.cuda()
    else:
        x_dev = torch.from_numpy(buf).cuda()
    q, qs, wo = _quantize(dtype, x32, x_dev, ld, w, c, fold)
    rq, rqs, rwo = oracle.quantize_query(dtype, x32, w, np.float32(c), fold=fold)
    assert np.array_equal(q, rq), "codes differ from the oracle"
    if rqs is None:
        assert qs is None
    else:
        assert np.array_equal(qs, rqs), "scales differ from the oracle"
    assert np.array_equal(wo.view(np.uint32), rwo.view(np.uint32)), "weights differ"


def test_quantize_query_weights_in_place_and_many_rows():
    """4099 rows (a ragged count of work groups), weights rewritten in place."""
    log("q quant 4099 rows in place")
    rng = np.random.default_rng(7)
    R = 4099
    x32 = (rng.standard_normal((R, 64, 128)) * 3).astype(np.float32)
    w = rng.standard_normal((R, 64)).astype(np.float32)
    q, _, wo = _quantize(synth.FP8, x32, torch.from_numpy(x32).cuda(), ROW, w, 0.5, True,
                         in_place=True)
    rq, _, rwo = oracle.quantize_query(synth.FP8, x32, w, np.float32(0.5), fold=True)
    assert np.array_equal(q, rq)
    assert np.array_equal(wo, rwo)


@pytest.mark.parametrize("dtype", [synth.FP8, synth.MXFP4])
def test_quantized_query_scores_like_the_oracle(dtype):
    """forward_pre's quantization followed by the paged scores and top-k: the
    GPU-quantized query (FP8 with the scale folded into the weights) scores
    within the logit tolerance of the oracle's scores of its own quantization
    of the same rows, and selects the same top-k apart from tolerance ties."""
    log("q quant then score dtype %d" % dtype)
    case = synth.decode_case([900, 3000, 17], next_n=1, P=64, dtype=dtype, k=256, seed=31,
                             canary=False)
    rng = np.random.default_rng(32)
    x32 = (rng.standard_normal((case.R, 64, 128))
           * np.exp2(rng.integers(-3, 4, size=(case.R, 64, 1)))).astype(np.float32)
    w = rng.standard_normal((case.R, 64)).astype(np.float32)
    c = np.float32(0.0625)
    fold = dtype == synth.FP8
    rq, rqs, rwo = oracle.quantize_query(dtype, x32, w, c, fold=fold)
    case.q, case.q_scale, case.w = rq, rqs, rwo
    dc = DeviceCase(case)
    # replace the uploaded query by the library's own quantization
    assert (dc.t["q_scale"] is None) == fold
    dc.t["q"].fill_(0)
    dc.t["w"].fill_(0)
    if not fold:
        dc.t["q_scale"].fill_(0)
    idx.idx_quantize_query(torch.from_numpy(x32).cuda(), idx.IDX_KIN_F32, ROW, case.R,
                           torch.from_numpy(w).cuda(), float(c), dc.query)
    logits, out, _ = run_decode(dc)
    ref, E = oracle_decode_rows(case, np.arange(case.R))
    for r in range(case.R):
        check_logits(logits[r].numpy(), ref[r], int(E[r]), "row %d" % r)
        check_topk_band(out[r].numpy(), ref[r], int(E[r]), case.k, "row %d" % r)
