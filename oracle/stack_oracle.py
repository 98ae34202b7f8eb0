"""Plain fp64 CPU oracle for a multi-layer decode step built around the
LongFlow operator (test infrastructure only).

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the library.  It
shares no code with the HIP implementation.

Source for the operator: "LongFlow: Efficient KV Cache Compression for
Reasoning Models" (arXiv 2603.11504); Figure 1 caption (the attention module
of a Qwen3-8B-shaped model at batch 128, length 3200) and Figure 2 caption
(one fused decode operator per attention call).  The pages do not describe
the layers around the operator.  Readings taken here, each the plainest one
for a Qwen3-8B-shaped attention module:

* one layer: qkv = x W_qkv^T (W_qkv rows are the Hq + 2 Hkv heads' output
  features, q first, then k, then v); q and the new k are rotated by RoPE
  at the sequence's position; the LongFlow decode step (decode_step) runs
  on q, the new k/v and the layer's cache; the layer output is
  x + O W_o^T (residual), with O the heads' outputs laid end to end.
* RoPE rotates the pairs (i, i + d/2), i < d/2, of every head by the angle
  pos * base^(-2i/d) (the "rotate half" layout); base 1e6 for Qwen3-8B.
* activations are bf16 between stages (qkv, rotated q/k, O, x), rounded to
  nearest even from the fp64 result through fp32 (the precision a GPU
  computes each stage in); every stage itself is evaluated in fp64.
* normalisation layers and the MLP are outside the attention module and are
  left out.
"""

import numpy as np

from .longflow_oracle import bf16_bits_to_f64, decode_step


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 bit patterns: first to float32 (nearest
    even, numpy's cast), then to bf16 by nearest even on the bit pattern.
    NaN stays a quiet NaN."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = np.ascontiguousarray(f).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[np.isnan(f)] = 0x7FC0
    return out


def rope(x, pos, base):
    """Rotate the (i, i + d/2) pairs of x [..., d] by pos * base^(-2i/d).

    pos broadcasts against x's leading dimensions without the last one.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = float(base) ** (-2.0 * np.arange(half) / d)              # [d/2]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv         # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def project(x_bits, w_bits):
    """x W^T in fp64 for bf16 x [M, K] and W [N, K]."""
    return bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(w_bits).T


def stack_step(x_bits, pos, layers, Hq, Hkv, d, scale, base):
    """One decode step through every layer.

    x_bits  uint16 [B, H]     bf16 input activations of the new token
    pos     int    [B]        its position in each sequence
    layers  list of dicts, one per layer, with
              w_qkv uint16 [(Hq + 2 Hkv) d, H], w_o uint16 [H, Hq d],
              k, v uint16 [B, Hkv, S, d] (updated in place),
              mask [B, S], slot int32 [B, Hkv] (the previous choice on entry,
              this step's evicted slot on return)
    Returns (x_out bits [B, H], per-layer list of (x_in bits, q bits, k_new
    bits, v_new bits, O fp64, scores, evict)).
    """
    B = x_bits.shape[0]
    x = np.asarray(x_bits, dtype=np.uint16)
    trace = []
    for lay in layers:
        qkv = f64_to_bf16_bits(project(x, lay["w_qkv"]))               # [B, (Hq+2Hkv) d]
        q = qkv[:, :Hq * d].reshape(B, Hq, d)
        kn = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(B, Hkv, d)
        vn = qkv[:, (Hq + Hkv) * d:].reshape(B, Hkv, d).copy()
        p = np.asarray(pos)[:, None]
        q = f64_to_bf16_bits(rope(bf16_bits_to_f64(q), p, base))
        kn = f64_to_bf16_bits(rope(bf16_bits_to_f64(kn), p, base))
        out, scores, evict = decode_step(q, lay["k"], lay["v"], lay["mask"], kn, vn, lay["slot"], scale)
        o_bits = f64_to_bf16_bits(out.reshape(B, Hq * d))
        x_next = f64_to_bf16_bits(bf16_bits_to_f64(x) + project(o_bits, lay["w_o"]))
        trace.append((x, q, kn, vn, out, scores, evict))
        lay["slot"][...] = evict
        x = x_next
    return x, trace
