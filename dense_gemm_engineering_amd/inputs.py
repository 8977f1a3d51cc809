"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the GEMM's arithmetic: it draws numbers, casts them
to the storage type with library casts (numpy's float16 cast and torch's CPU
bfloat16 cast, both round-to-nearest-even) and packs q4 blocks in their
storage format.  The same host arrays feed both the GPU library and the CPU
oracle.

Seeds: operand o of workload w, variant v, uses PCG64(1000*w + 10*v + o), with
o = 1 (A), 2 (B), 3 (bias), 4 (q4 scales), 5 (q4 codes), 6 (old C).

Workloads (all row-major; w is the seed family):
  square256 (w=1)          256^3 fp16, U[-1,1); a second pass with integers
                           in [-4, 4]
  square4096 (w=2)         4096^3 fp16 or bf16, N(0,1)/sqrt(K)
  fp32_square (w=3)        n^3 fp32, U[-1,1), n in {1024, 2048, 4096}
  prefill_projection (w=4) A 2048 x K fp16 N(0,1); W N x K as q4 blocks with
                           scales fp16(|N(0, 0.02)|) and codes uniform 0..15
  tall_skinny (w=5)        X 65536 x 160 and W 160 x N (N = 160 or 32), both
                           N(0,1)/sqrt(160) fp16; bias fp16 N(0, 0.1)
  decode_shape (w=6)       X M x 4096 fp16 N(0,1), M in {1, 8, 16, 32, 64}; one
                           4096 x 4096 (N x K) fp16 weight N(0,1)/sqrt(4096)
  kquant_projection (w=7)  prefill_projection's A and shapes with the weight in
                           a 256-weight super-block format (q4_k, q6_k or
                           q6_k at a 224-byte stride):
                           every byte uniform, then each binary16 scale
                           field overwritten with fp16(|N(0, s)|) (q6_k d:
                           s = 2e-5; q4_k d and dmin: s = 4e-5), so weights
                           are of the q4 workload's magnitude
"""
import numpy as np

OP_A, OP_B, OP_BIAS, OP_SCALE, OP_CODE, OP_C = 1, 2, 3, 4, 5, 6


def seed(workload, operand, variant=0):
    return 1000 * workload + 10 * variant + operand


def rng(workload, operand, variant=0):
    return np.random.Generator(np.random.PCG64(seed(workload, operand, variant)))


def to_bits(x, dtype):
    """float64 array -> raw storage bits (uint16 for f16/bf16, uint32 for f32)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "f32":
        return x.astype(np.float32).view(np.uint32)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def uniform(shape, dtype, workload, operand, variant=0, lo=-1.0, hi=1.0):
    return to_bits(rng(workload, operand, variant).uniform(lo, hi, size=shape), dtype)


def normal(shape, dtype, workload, operand, variant=0, std=1.0):
    return to_bits(rng(workload, operand, variant).standard_normal(size=shape) * std, dtype)


def integers(shape, dtype, workload, operand, variant=0, lo=-4, hi=4):
    """Integer-valued entries in [lo, hi] (inclusive)."""
    v = rng(workload, operand, variant).integers(lo, hi + 1, size=shape).astype(np.float64)
    return to_bits(v, dtype)


def pack_q4(scale_bits, codes):
    """Pack q4 blocks: scale_bits (rows, nb) uint16, codes (rows, nb, 32) in 0..15.

    Each block is 18 bytes: the scale, little-endian, then 16 bytes whose low
    nibble is element i and high nibble element i + 16.
    """
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    codes = np.asarray(codes, dtype=np.uint8)
    rows, nb = scale_bits.shape
    assert codes.shape == (rows, nb, 32)
    blk = np.empty((rows, nb, 18), dtype=np.uint8)
    blk[:, :, 0] = (scale_bits & 0xFF).astype(np.uint8)
    blk[:, :, 1] = (scale_bits >> 8).astype(np.uint8)
    blk[:, :, 2:] = codes[:, :, :16] | (codes[:, :, 16:] << 4)
    return blk.reshape(-1)


def q4_weights(rows, cols, workload=4, variant=0, scale_std=0.02):
    """Synthetic q4 weight matrix (rows x cols) as raw block bytes."""
    assert cols % 32 == 0
    nb = cols // 32
    d = np.abs(rng(workload, OP_SCALE, variant).standard_normal(size=(rows, nb)) * scale_std)
    scale_bits = to_bits(d, "f16")
    codes = rng(workload, OP_CODE, variant).integers(0, 16, size=(rows, nb, 32))
    return pack_q4(scale_bits, codes)


# Super-block formats: (weights, bytes, byte offsets of the binary16 scale
# fields, scale std)
KQUANT = {"q4_k": (256, 144, (0, 2), 4e-5), "q6_k": (256, 210, (208,), 2e-5),
          "q6_k_224": (256, 224, (208,), 2e-5)}


def kquant_weights(qtype, rows, cols, workload=7, variant=0):
    """Synthetic rows x cols weight in a super-block format: uniform random
    bytes (codes, sub-block scales and mins) with sane binary16 scales."""
    w, nbytes, offs, std = KQUANT[qtype]
    assert cols % w == 0
    nsb = rows * (cols // w)
    q = rng(workload, OP_CODE, variant).integers(0, 256, size=(nsb, nbytes), dtype=np.uint8)
    r = rng(workload, OP_SCALE, variant)
    for off in offs:
        bits = to_bits(np.abs(r.standard_normal(nsb) * std), "f16")
        q[:, off] = bits & 0xFF
        q[:, off + 1] = bits >> 8
    return q.reshape(-1)


def kquant_projection(qtype, shape="up", M=2048):
    """prefill_projection with the weight as super-blocks: A, q, N, K."""
    N, K = PREFILL_SHAPES[shape]
    v = {"up": 0, "attn": 1, "down": 2}[shape]
    A = normal((M, K), "f16", 4, OP_A, v)
    q = kquant_weights(qtype, N, K, 7, v + {"q4_k": 0, "q6_k": 3, "q6_k_224": 6}[qtype])
    return A, q, N, K


# ----------------------------------------------------------------- workloads

def square256(integer=False):
    if integer:
        return (integers((256, 256), "f16", 1, OP_A, 1), integers((256, 256), "f16", 1, OP_B, 1))
    return uniform((256, 256), "f16", 1, OP_A), uniform((256, 256), "f16", 1, OP_B)


def square4096(dtype="f16", n=4096):
    s = 1.0 / np.sqrt(n)
    return (normal((n, n), dtype, 2, OP_A, std=s), normal((n, n), dtype, 2, OP_B, std=s))


def fp32_square(n):
    v = {1024: 0, 2048: 1, 4096: 2}.get(n, 3)
    return uniform((n, n), "f32", 3, OP_A, v), uniform((n, n), "f32", 3, OP_B, v)


PREFILL_SHAPES = {"up": (11008, 4096), "attn": (4096, 4096), "down": (4096, 11008)}


def prefill_projection(shape="up", M=2048):
    """Prefill projection inputs: A (M x K fp16 bits), q4 weight bytes, N, K."""
    N, K = PREFILL_SHAPES[shape]
    v = {"up": 0, "attn": 1, "down": 2}[shape]
    A = normal((M, K), "f16", 4, OP_A, v)
    q = q4_weights(N, K, 4, v)
    return A, q, N, K


DECODE_ROWS = (1, 8, 16, 32, 64)


def decode_shape(M=1, N=4096, K=4096):
    """Decode-shaped inputs: X (M x K) fp16 N(0,1) and an N x K fp16 weight
    N(0,1)/sqrt(K) (one 4096 x 4096 layer times M input vectors)."""
    v = DECODE_ROWS.index(M) if M in DECODE_ROWS else 9
    X = normal((M, K), "f16", 6, OP_A, v)
    W = normal((N, K), "f16", 6, OP_B, 0, std=1.0 / np.sqrt(K))
    return X, W


def tall_skinny(N=160, M=65536, K=160):
    v = 0 if N == 160 else 1
    s = 1.0 / np.sqrt(K)
    X = normal((M, K), "f16", 5, OP_A, v, std=s)
    W = normal((K, N), "f16", 5, OP_B, v, std=s)
    bias = normal((N,), "f16", 5, OP_BIAS, v, std=0.1)
    return X, W, bias
