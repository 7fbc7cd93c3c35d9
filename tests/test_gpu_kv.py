"""GPU parity of the low-bit KV cache (w4a4_kv_quant / w4a4_kv_dequant
through the C ABI) against the oracle's kv_quantize / kv_dequantize: the
cache bytes and scales of every written slot bit-exact, untouched slots
unchanged, and the gathered fp16 bit-exact. Atom summary page, Summary
paragraph 2 (low bit-width KV cache); per-block quantization as in the NQKV
abstract on the "smoothquant" tag page.
"""
import sys

import numpy as np
import pytest

import mixed_precision_integer_amd as w4

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    sys.stderr.write(f"\n[gpu case] {msg}\n")
    sys.stderr.flush()


def draw(T, H, D, seed):
    rng = np.random.default_rng(seed)
    scale = rng.choice([2.0 ** -10, 0.05, 1.0, 30.0], (T, H, 1))
    X = (rng.standard_normal((T, H, D)) * scale).astype(np.float16)
    X[0, 0] = 0                                   # an all-zero head: scale 0, codes 0
    return X


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("bits", [4, 8])
def test_kv_parity(oracle, D, bits):
    T, H, num_slots = 37, 6, 64
    _say(f"kv D={D} bits={bits}")
    X = draw(T, H, D, seed=D + bits)
    rng = np.random.default_rng(D * bits)
    slots = rng.permutation(num_slots)[:T].astype(np.int32)
    slots[3] = -1                                  # padding token: skipped
    slots[7] = num_slots + 5                       # outside the cache: skipped
    cache = w4.KVCache(num_slots, H, D, bits, DEV)
    sd = torch.from_numpy(slots).to(DEV)
    cache.store(torch.from_numpy(X.reshape(T, H * D)).to(DEV), sd)
    Y = cache.load(sd)
    q, s = oracle.kv_quantize(X, bits)
    packed = oracle.kv_pack(q, bits)
    want_y = oracle.kv_dequantize(q, s)
    cq, cs = cache.q.cpu().numpy(), cache.s.cpu().numpy()
    yv = Y.cpu().numpy().reshape(T, H, D)
    valid = (slots >= 0) & (slots < num_slots)
    for t in range(T):
        if valid[t]:
            assert np.array_equal(cq[slots[t]], packed[t]), f"codes of token {t}"
            assert np.array_equal(cs[slots[t]].view(np.uint32), s[t].view(np.uint32)), f"scales of token {t}"
            assert np.array_equal(yv[t].view(np.uint16), want_y[t].view(np.uint16)), f"gather of token {t}"
        else:
            assert np.all(yv[t].view(np.uint16) == 0), f"invalid slot of token {t} reads as zeros"
    untouched = np.setdiff1d(np.arange(num_slots), slots[valid])
    assert np.all(cq[untouched] == 0) and np.all(cs[untouched] == 0)


def test_kv_identity_slots_and_pitch(oracle):
    """No slot mapping (slot = token) and a row pitch larger than H * D."""
    T, H, D, bits = 50, 3, 128, 4
    _say("kv identity slots")
    X = draw(T, H, D, seed=3)
    buf = torch.zeros((T, H * D + 40), dtype=torch.float16, device=DEV)
    buf[:, :H * D] = torch.from_numpy(X.reshape(T, H * D)).to(DEV)
    cache = w4.KVCache(T, H, D, bits, DEV)
    cache.store(buf[:, :H * D])
    Y = cache.load(T=T)
    q, s = oracle.kv_quantize(X, bits)
    torch.cuda.synchronize()
    assert np.array_equal(cache.q.cpu().numpy(), oracle.kv_pack(q, bits))
    assert np.array_equal(Y.cpu().numpy().reshape(T, H, D).view(np.uint16),
                          oracle.kv_dequantize(q, s).view(np.uint16))


@pytest.mark.parametrize("bits", [4, 8])
def test_kv_full_size(oracle, bits):
    """A 65B-style cache append: 4096 tokens x 64 heads x 128 channels."""
    T, H, D = 4096, 64, 128
    _say(f"kv full size bits={bits}")
    X = draw(T, H, D, seed=11 + bits)
    slots = np.random.default_rng(5).permutation(2 * T)[:T].astype(np.int32)
    cache = w4.KVCache(2 * T, H, D, bits, DEV)
    sd = torch.from_numpy(slots).to(DEV)
    cache.store(torch.from_numpy(X.reshape(T, H * D)).to(DEV), sd)
    Y = cache.load(sd)
    q, s = oracle.kv_quantize(X, bits)
    torch.cuda.synchronize()
    assert np.array_equal(cache.q.cpu().numpy()[slots], oracle.kv_pack(q, bits))
    assert np.array_equal(cache.s.cpu().numpy()[slots].view(np.uint32), s.view(np.uint32))
    assert np.array_equal(Y.cpu().numpy().reshape(T, H, D).view(np.uint16),
                          oracle.kv_dequantize(q, s).view(np.uint16))
