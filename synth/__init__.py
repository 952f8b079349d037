"""Seeded synthetic inputs for the block-quantized matmul workloads.

Shared by the oracle tests, the GPU parity tests and the bench.  It only draws random bytes and
numbers and places them in the block byte layouts; it holds none of the method's arithmetic
(no quantization, no decoding, no dot products).

Value distributions (the workload descriptions give Q4_K's; the rest are the plainest readings):
  * Q4_K super-block (144 B): fp16 d and dmin ~ U(0.001, 0.02); 12 bytes of uniform random
    6-bit-packed scales/mins; 128 bytes of uniform random nibbles.
  * Q5_K super-block (176 B): as Q4_K, with 32 bytes of uniform random fifth bits (qh).
  * Q4_0 block (18 B): fp16 d ~ U(0.001, 0.02), 16 bytes of uniform random nibbles.
  * Q6_K super-block (210 B): uniform random ql (128 B) and qh (64 B); int8 scales ~ U{-32..31};
    fp16 d ~ U(0.001, 0.02).
  * Q8_0 block (34 B): fp16 d ~ U(0.001, 0.02); int8 codes ~ U{-127..127}.
  * Q3_K super-block (110 B): uniform random hmask (32 B), qs (64 B) and 6-bit-packed scales
    (12 B); fp16 d ~ U(0.001, 0.02).
  * IQ4_XS super-block (136 B): fp16 d ~ U(0.001, 0.02); uniform random scale bits (2 + 4 B) and
    4-bit codebook indices (128 B).
  * Activations: N(0, 1) fp32.
  * MoE routing: expert e has probability proportional to (e + 1)^-s; each token draws top_k
    distinct experts by successive sampling without replacement.
fp16 values are produced by numpy's float32 -> float16 cast.
"""
import numpy as np

Q8_0 = 8
Q4_0 = 2
Q4_K = 12
Q5_K = 13
Q6_K = 14
Q3_K = 11
IQ4_XS = 23
TYPE_NAMES = {Q4_0: "q4_0", Q8_0: "q8_0", Q4_K: "q4_K", Q5_K: "q5_K", Q6_K: "q6_K", Q3_K: "q3_K", IQ4_XS: "iq4_xs"}
BLOCK_VALUES = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, Q3_K: 256, IQ4_XS: 256}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210, Q3_K: 110, IQ4_XS: 136}


def rngs(seed, n):
    """n independent generators from one seed."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _fp16_bytes(vals):
    return np.ascontiguousarray(vals.astype(np.float32).astype(np.float16)).view(np.uint8).reshape(
        vals.shape + (2,))


def gen_weights(qtype, rows, k, rng):
    """uint8 [rows, k/QK * block_bytes] random blocks of the given type."""
    qk = BLOCK_VALUES[qtype]
    bb = BLOCK_BYTES[qtype]
    assert k % qk == 0
    nb = rows * (k // qk)
    blk = rng.integers(0, 256, size=(nb, bb), dtype=np.uint8)
    if qtype in (Q4_K, Q5_K):
        blk[:, 0:2] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
        blk[:, 2:4] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
    elif qtype == Q6_K:
        blk[:, 192:208] = rng.integers(-32, 32, size=(nb, 16)).astype(np.int8).view(np.uint8)
        blk[:, 208:210] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
    elif qtype == Q4_0:
        blk[:, 0:2] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
    elif qtype == Q8_0:
        blk[:, 0:2] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
        blk[:, 2:34] = rng.integers(-127, 128, size=(nb, 32)).astype(np.int8).view(np.uint8)
    elif qtype == Q3_K:
        blk[:, 108:110] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
    elif qtype == IQ4_XS:
        blk[:, 0:2] = _fp16_bytes(rng.uniform(0.001, 0.02, size=nb))
    else:
        raise ValueError(qtype)
    return blk.reshape(rows, (k // qk) * bb)


def gen_activations(n, k, rng):
    return rng.standard_normal((n, k), dtype=np.float32)


def zipf_probs(n_exp, s):
    p = (np.arange(n_exp, dtype=np.float64) + 1.0) ** (-s)
    return p / p.sum()


def gen_routing(n_tok, top_k, n_exp, s, rng):
    """int32 [n_tok, top_k] expert ids, distinct within a token."""
    p = zipf_probs(n_exp, s)
    ids = np.empty((n_tok, top_k), dtype=np.int32)
    for t in range(n_tok):
        ids[t] = rng.choice(n_exp, size=top_k, replace=False, p=p)
    return ids


# ------------------------------------------------------------------------------------------------
# The workloads.  Each entry is a plain description; make_* builds the arrays with seed 0.
# ------------------------------------------------------------------------------------------------
DENSE_SMALL = dict(name="q4_K 512x1024 x 16 tokens", qtype=Q4_K, rows=512, k=1024, n=16)

MMVQ_CASES = [dict(name=f"{TYPE_NAMES[t]} 4096x4096 N={n}", qtype=t, rows=4096, k=4096, n=n)
              for t in (Q4_K, Q6_K, Q8_0) for n in (1, 2, 5, 8)]

PREFILL_CASES = [
    dict(name="ffn up q4_K 14336x4096 T=512", qtype=Q4_K, rows=14336, k=4096, n=512),
    dict(name="ffn down q6_K 4096x14336 T=512", qtype=Q6_K, rows=4096, k=14336, n=512),
    dict(name="ffn up q4_K 14336x4096 T=2048", qtype=Q4_K, rows=14336, k=4096, n=2048),
    dict(name="ffn down q6_K 4096x14336 T=2048", qtype=Q6_K, rows=4096, k=14336, n=2048),
]

MOE_CASES = [
    dict(name="moe 8x q4_K 14336x4096, 512 tok top-2 zipf1.1", qtype=Q4_K, n_exp=8, rows=14336,
         k=4096, n_tok=512, top_k=2, zipf=1.1, x_per_tok=1),
    dict(name="moe 128x q4_K 768x2048 gate/up, 2048 tok top-8 zipf1.0", qtype=Q4_K, n_exp=128,
         rows=768, k=2048, n_tok=2048, top_k=8, zipf=1.0, x_per_tok=1),
    dict(name="moe 128x q6_K 2048x768 down, 2048 tok top-8 zipf1.0", qtype=Q6_K, n_exp=128,
         rows=2048, k=768, n_tok=2048, top_k=8, zipf=1.0, x_per_tok=8),
    dict(name="moe 128x q4_K 768x2048 gate/up, 64 tok top-8 zipf1.0 (sparse experts)", qtype=Q4_K,
         n_exp=128, rows=768, k=2048, n_tok=64, top_k=8, zipf=1.0, x_per_tok=1),
]


# Q5_K, Q4_0, Q3_K and IQ4_XS (beyond the headline types): the matrix-vector shapes and one prefill
# shape each.
EXTRA_MMVQ_CASES = [dict(name=f"{TYPE_NAMES[t]} 4096x4096 N={n}", qtype=t, rows=4096, k=4096, n=n)
                    for t in (Q5_K, Q4_0, Q3_K, IQ4_XS) for n in (1, 2, 5, 8)]
EXTRA_PREFILL_CASES = [dict(name=f"ffn up {TYPE_NAMES[t]} 14336x4096 T=512", qtype=t, rows=14336, k=4096, n=512)
                       for t in (Q5_K, Q4_0, Q3_K, IQ4_XS)]

# Gate/up products fused with SwiGLU: two matrices of `rows` rows each.
GLU_CASES = [
    dict(name="ffn gate/up+swiglu q4_K 2x14336x4096 N=1", kind="dense", qtype=Q4_K, rows=14336, k=4096, n=1),
    dict(name="ffn gate/up+swiglu q4_K 2x14336x4096 T=512", kind="dense", qtype=Q4_K, rows=14336, k=4096, n=512),
    dict(name="moe 128x gate/up+swiglu q4_K 2x768x2048, 2048 tok top-8 zipf1.0", kind="moe", qtype=Q4_K,
         n_exp=128, rows=768, k=2048, n_tok=2048, top_k=8, zipf=1.0, x_per_tok=1),
]


def make_glu(case, seed=0):
    """(w_gate, w_up, x, ids or None) of a GLU case."""
    if case["kind"] == "dense":
        g_g, g_u, g_x = rngs(seed, 3)
        return (gen_weights(case["qtype"], case["rows"], case["k"], g_g),
                gen_weights(case["qtype"], case["rows"], case["k"], g_u),
                gen_activations(case["n"], case["k"], g_x), None)
    g_g, g_u, g_x, g_r = rngs(seed, 4)
    nr = case["n_exp"] * case["rows"]
    return (gen_weights(case["qtype"], nr, case["k"], g_g), gen_weights(case["qtype"], nr, case["k"], g_u),
            gen_activations(case["n_tok"], case["k"], g_x),
            gen_routing(case["n_tok"], case["top_k"], case["n_exp"], case["zipf"], g_r))


def make_dense(case, seed=0):
    g_w, g_x = rngs(seed, 2)
    w = gen_weights(case["qtype"], case["rows"], case["k"], g_w)
    x = gen_activations(case["n"], case["k"], g_x)
    return w, x


def make_moe(case, seed=0):
    g_w, g_x, g_r = rngs(seed, 3)
    w = gen_weights(case["qtype"], case["n_exp"] * case["rows"], case["k"], g_w)
    x = gen_activations(case["n_tok"] * case["x_per_tok"], case["k"], g_x)
    ids = gen_routing(case["n_tok"], case["top_k"], case["n_exp"], case["zipf"], g_r)
    return w, x, ids
