"""GPU parity of FP8 (OCP E4M3) embedding slabs against the FP8 oracle.

Tokens, selected centroids, masked logits and the fused top-m must match the
oracle bit for bit; the quantisation happens on the GPU at prepare time, so
every comparison also checks the codes and scales it produced.
"""

import numpy as np
import pytest

from oracle import fp8_slabs as f8
from oracle import top_tokens as top_tokens_bf16
from tests.gpu_helpers import rows, to_device, torch_mod
from workloads import make_random, make_workload

pytestmark = pytest.mark.gpu


def _head(w, max_B, max_K=None):
    from centroid_masked_sparse_amd import Head
    equal = np.all(np.diff(w.offsets) == w.V // w.Nc) and w.V % w.Nc == 0
    return Head(to_device(w.C, w.dtype), to_device(w.E, w.dtype), w.tos,
                None if equal else w.offsets, max_B=max_B,
                max_K=max_K if max_K is not None else w.Nc, slabs="fp8")


def _check_all(head, w, B, K, m=6):
    torch = torch_mod()
    hb = rows(w, B)
    h = to_device(hb, w.dtype)
    codes, sc = f8.quantize_rows(w.E)
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(h, K, topk_out=tk)
    masked = head.masked_logits(h, K)
    tm, vm = head.top_m(h, m, K)
    torch.cuda.synchronize()
    tok_o, sel_o = f8.top_tokens_fp8(hb, w.C, codes, sc, w.offsets, w.tos, K)
    assert tk.cpu().numpy().tolist() == sel_o.tolist()
    assert tok.cpu().numpy().tolist() == tok_o.tolist(), (B, K)
    M = f8.masked_logits_fp8(hb, w.C, codes, sc, w.offsets, w.tos, K)
    assert np.array_equal(masked.cpu().numpy().view(np.uint32), M.view(np.uint32))
    tm_o, vm_o = f8.top_m_fp8(hb, w.C, codes, sc, w.offsets, w.tos, K, m)
    assert tm.cpu().numpy().tolist() == tm_o.tolist()
    assert np.array_equal(vm.cpu().numpy().view(np.uint32), vm_o.view(np.uint32))


@pytest.mark.parametrize("seed,d,V,Nc,K,B,ragged", [
    (61, 128, 8192, 64, 4, 9, False),
    (62, 64, 3000, 40, 3, 7, True),       # ragged clusters, some tiny or empty
    (63, 256, 16384, 256, 16, 64, False),
    (64, 512, 5000, 50, 2, 70, True),     # two passes of rows
    (65, 320, 4096, 64, 5, 5, False),     # d with no straight-line pipeline
    (67, 128, 8192, 64, 8, 40, False),    # B*K > 2*Nc below 48 rows: masked and top-m on the unsplit tile grid
])
def test_random_shapes(seed, d, V, Nc, K, B, ragged):
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    _check_all(_head(w, max_B=B), w, B, K)


def test_every_code_and_zero_rows():
    """Rows holding every finite E4M3 value with 448 as the maximum get scale
    1, so their codes are exact: the logits then depend on every code's
    hardware decode.  Zero rows get scale 1 and zero codes; rows of tiny
    values land in the subnormal codes."""
    from workloads.synth import f32_to_bf16_bits
    rng = np.random.default_rng(66)
    d, Nc, vpc = 128, 16, 64
    V = Nc * vpc
    w = make_random(66, d=d, V=V, Nc=Nc, dtype="bf16", rows=8)
    vals = f8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    allv = np.concatenate([vals, -vals])                       # 254 values incl. +-0
    E = w.E.copy()
    for j in range(0, V, 3):
        r = rng.permutation(allv)[:d]
        r[rng.integers(d)] = 448.0
        E[j] = f32_to_bf16_bits(r.astype(np.float32))
    E[1] = 0
    E[4] = f32_to_bf16_bits((rng.standard_normal(d) * 1e-30).astype(np.float32))
    w2 = type(w)(w.name, w.seed, d, V, Nc, 4, "bf16", w.h, w.C, E, w.offsets, w.tos)
    _check_all(_head(w2, max_B=8), w2, 8, 4, m=32)
    _check_all(_head(w2, max_B=8), w2, 8, Nc, m=32)           # every slot is a candidate


def test_sweep_config_full_size():
    """The sweep head (d=256, V=262144, Nc=2048, K=32) with FP8 slabs at
    B=64: every token against the oracle, quantising only the rows the
    selected clusters own (the selection does not depend on the slabs).
    Also reports how often the FP8 argmax equals the bf16 one."""
    torch = torch_mod()
    w = make_workload("sweep")
    B, K = 64, w.K
    head = _head(w, max_B=B, max_K=K)
    hb = rows(w, B)
    tok = head.top_tokens(to_device(hb, w.dtype), K)
    torch.cuda.synchronize()
    tok_b, sel, _ = top_tokens_bf16(hb, w.C, w.E, w.offsets, w.tos, K, w.dtype)
    used = np.unique(np.concatenate([np.arange(w.offsets[c], w.offsets[c + 1])
                                     for c in np.unique(sel)]))
    codes = np.zeros((w.V, w.d), dtype=np.uint8)
    sc = np.ones(w.V, dtype=np.float32)
    codes[used], sc[used] = f8.quantize_rows(w.E[used])
    tok_o, sel_o = f8.top_tokens_fp8(hb, w.C, codes, sc, w.offsets, w.tos, K)
    assert np.array_equal(sel_o, sel)
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    agree = float(np.mean(tok_o == tok_b))
    print(f"FP8 argmax equals the bf16 argmax on {agree:.3f} of the rows")
    assert agree > 0.5


def test_fp8_requires_bf16():
    from centroid_masked_sparse_amd import CeError, Head
    torch = torch_mod()
    C = torch.zeros((4, 64), dtype=torch.float32, device="cuda:0")
    E = torch.zeros((256, 64), dtype=torch.float32, device="cuda:0")
    with pytest.raises(CeError):
        Head(C, E, np.arange(256), max_B=2, slabs="fp8")


def test_draft_step_with_fp8_slabs():
    """The fused draft step runs on an FP8 head: its tokens are the FP8
    oracle's tokens of the normalised rows."""
    from oracle import draft as od
    from workloads.synth import f32_to_bf16_bits
    torch = torch_mod()
    w = make_random(67, d=256, V=8192, Nc=64, dtype="bf16", rows=16)
    head = _head(w, max_B=16)
    rng = np.random.default_rng(67)
    x = f32_to_bf16_bits((2.0 * rng.standard_normal((16, 256))).astype(np.float32))
    nw = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(256)).astype(np.float32))
    h, tok, _ = head.draft_step(to_device(x, "bf16"), to_device(nw, "bf16"), 1e-6, 4)
    torch.cuda.synchronize()
    hn = od.rms_norm(x, nw, 1e-6, "bf16")
    codes, sc = f8.quantize_rows(w.E)
    tok_o, _ = f8.top_tokens_fp8(hn, w.C, codes, sc, w.offsets, w.tos, 4)
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
