"""Seeded synthetic inputs in the library's host formats.

This module draws random numbers and packs them into the byte layouts that
``il_upload`` accepts.  It holds none of the layer's arithmetic (no decoding,
no products, no sums), so the GPU path and the CPU oracle can both be fed
from it without sharing any of the computation they are compared on.

Workloads stand in for the pages' real-checkpoint decode / verify / prefill
traffic (linear layers of a transformer called with one shared input, see the
``Drafter::step`` listing on the oxinfer 0.0.1 ``src/drafter.rs`` page): the
checkpoints are not available, so tensors are drawn from fixed distributions:

  x          f32 ~ N(0, 1)
  bf16 W     f32 ~ N(0, 0.02), rounded to bfloat16 (round-to-nearest-even)
  Q8 W       int8 codes uniform in [-127, 127]; f32 block scales ~ U[1e-4, 1e-3]
  Q4 W       4-bit codes uniform in 0..15 (value (q - 8) * scale); f16 block
             scales ~ U[1e-3, 1e-2] (rounded to binary16 by numpy)

Every tensor comes from ``numpy.random.Generator(PCG64(SeedSequence([cfg,
tensor_id])))``: tensor_id 0 is the shared x, j >= 1 is job j (codes drawn
before scales), 99 is the separate input of the 14336-wide Q8 job.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

BF16, Q8, Q4 = 0, 1, 2
FMT_NAMES = {BF16: "bf16", Q8: "q8", Q4: "q4"}
BLOCK = 32
Q8_BLOCK_BYTES = 36  # float32 scale + 32 int8 codes
Q4_BLOCK_BYTES = 18  # f16 scale bits + 16 bytes of nibbles


def weight_bytes(fmt: int, n_out: int, n_in: int) -> int:
    """Host-format storage of one weight: the byte count the GB/s metric uses."""
    if fmt == BF16:
        return 2 * n_out * n_in
    if fmt == Q8:
        return Q8_BLOCK_BYTES * n_out * (n_in // BLOCK)
    if fmt == Q4:
        return Q4_BLOCK_BYTES * n_out * (n_in // BLOCK)
    raise ValueError(f"unknown format {fmt}")


def rng_for(cfg: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tensor_id])))


# ----------------------------------------------------------------- encoders
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite f32 values to bfloat16 bit patterns (nearest, ties to even)."""
    # finite patterns stay below 2^32 after the rounding increment
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def encode_q8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Pack int8 codes [n_out, n_in] and f32 scales [n_out, n_in/32] into 36-byte
    blocks {f32 scale (LE); int8 q[32]}, row-major by (row, block)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n_out, n_in = codes.shape
    nb = n_in // BLOCK
    scales = np.ascontiguousarray(scales, dtype="<f4").reshape(n_out, nb)
    out = np.empty((n_out, nb, Q8_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, :4] = scales.view(np.uint8).reshape(n_out, nb, 4)
    out[:, :, 4:] = codes.view(np.uint8).reshape(n_out, nb, BLOCK)
    return out.reshape(-1)


def encode_q4(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [n_out, n_in] (0..15) and f16 scale bit patterns
    [n_out, n_in/32] into 18-byte blocks {u16 scale (LE); u8 qs[16]} where
    qs[j] = code[2j] | code[2j+1] << 4."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if codes.size and codes.max() > 15:
        raise ValueError("Q4 codes must be in 0..15")
    n_out, n_in = codes.shape
    nb = n_in // BLOCK
    scale_bits = np.ascontiguousarray(scale_bits, dtype="<u2").reshape(n_out, nb)
    pairs = codes.reshape(n_out, nb, BLOCK // 2, 2)
    out = np.empty((n_out, nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, :2] = scale_bits.view(np.uint8).reshape(n_out, nb, 2)
    out[:, :, 2:] = pairs[..., 0] | (pairs[..., 1] << 4)
    return out.reshape(-1)


# --------------------------------------------------------------- generators
def gen_x(cfg: int, tensor_id: int, rows: int, n_in: int) -> np.ndarray:
    return rng_for(cfg, tensor_id).standard_normal((rows, n_in), dtype=np.float32)


def gen_bf16(cfg: int, tensor_id: int, n_out: int, n_in: int) -> np.ndarray:
    g = rng_for(cfg, tensor_id)
    w = g.standard_normal((n_out, n_in), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(w)


def gen_f32_weight(cfg: int, tensor_id: int, n_out: int, n_in: int) -> np.ndarray:
    """Full-precision weights for the upload quantiser: f32 ~ N(0, 0.02), the
    bf16 weights' distribution before rounding."""
    g = rng_for(cfg, tensor_id)
    return g.standard_normal((n_out, n_in), dtype=np.float32) * np.float32(0.02)


# Upload-quantiser workloads (f32 [n_out, n_in] -> Q8 / Q4 on the device):
# the Q8 gate/up shape and the Q4 verify shape, one weight each.
QUANTIZE = {
    "f2_q8": (Q8, 14336, 4096, 6, 1),  # fmt, n_out, n_in, cfg, tensor_id
    "f2_q4": (Q4, 17408, 5120, 6, 2),
}


# Fused gate/up + GELU workloads (il_matmul_gelu_mul): the gate/up pair of the
# Q8 decode shape, and the same pair as Q4 and bf16; t = 1 (one drafted token),
# and the Q8 / Q4 pair at t = 512 (the prefill GEMM's gate/up mode).
GELU_MUL = {
    "f3_q8_t1": (Q8, 14336, 4096, 1, 7),  # fmt, n_out, n_in, t, cfg
    "f3_q4_t1": (Q4, 14336, 4096, 1, 7),
    "f3_bf16_t1": (BF16, 14336, 4096, 1, 7),
    "f3_q8_t512": (Q8, 14336, 4096, 512, 7),
    "f3_q4_t512": (Q4, 14336, 4096, 512, 7),
}


def make_gelu_mul_inputs(name: str):
    """(x [t, n_in] f32, gate, up) host-format weights of a GELU_MUL workload."""
    fmt, n_out, n_in, t, cfg = GELU_MUL[name]
    x = np.ascontiguousarray(gen_x(cfg, 0, t, n_in))
    return x, gen_weight(fmt, cfg, 1, n_out, n_in), gen_weight(fmt, cfg, 2, n_out, n_in)


# Centroid-masked LM head workload: a 256-wide drafter hidden state, 2048
# centroids, the top 32 visited, a vocabulary of 2^18 tokens (the pages state
# H, C and k; no vocabulary size, so 2^18 stands for a current LLM's).
LM_HEAD = {"f4_lmhead_t1": (256, 2048, 32, 1 << 18, 1, 8)}  # h, C, k, V, t, cfg


def make_lm_head_inputs(name: str):
    """(x [t, h] f32, centroids bf16 bits [C, h], embed bf16 bits [V, h],
    ordering uint32 [V]): N(0, 1) x, N(0, 0.02) rows, a seeded permutation."""
    h, n_c, k, vocab, t, cfg = LM_HEAD[name]
    x = np.ascontiguousarray(gen_x(cfg, 0, t, h))
    cen = gen_bf16(cfg, 1, n_c, h)
    emb = gen_bf16(cfg, 2, vocab, h)
    order = rng_for(cfg, 3).permutation(vocab).astype(np.uint32)
    return x, cen, emb, order


def gen_q8_parts(cfg: int, tensor_id: int, n_out: int, n_in: int):
    g = rng_for(cfg, tensor_id)
    codes = g.integers(-127, 128, size=(n_out, n_in), dtype=np.int8)
    scales = g.uniform(1e-4, 1e-3, size=(n_out, n_in // BLOCK)).astype(np.float32)
    return codes, scales


def gen_q4_parts(cfg: int, tensor_id: int, n_out: int, n_in: int):
    g = rng_for(cfg, tensor_id)
    codes = g.integers(0, 16, size=(n_out, n_in), dtype=np.uint8)
    scales = g.uniform(1e-3, 1e-2, size=(n_out, n_in // BLOCK)).astype(np.float16)
    return codes, scales.view(np.uint16)


def gen_weight(fmt: int, cfg: int, tensor_id: int, n_out: int, n_in: int) -> np.ndarray:
    """Host-format weight bytes (bf16: uint16 [n_out, n_in]; Q8/Q4: flat uint8)."""
    if fmt == BF16:
        return gen_bf16(cfg, tensor_id, n_out, n_in)
    if fmt == Q8:
        return encode_q8(*gen_q8_parts(cfg, tensor_id, n_out, n_in))
    if fmt == Q4:
        return encode_q4(*gen_q4_parts(cfg, tensor_id, n_out, n_in))
    raise ValueError(f"unknown format {fmt}")


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]


# ------------------------------------------------------------------ configs
@dataclass(frozen=True)
class Job:
    fmt: int
    n_out: int
    tensor_id: int


@dataclass(frozen=True)
class Submission:
    """One il_matmul call: jobs sharing x[:t] of the tensor (cfg, x_id)."""
    name: str
    cfg: int
    t: int
    n_in: int
    x_id: int
    x_rows: int  # rows drawn for that x tensor (t <= x_rows; smaller t take the first rows)
    jobs: tuple = field(default_factory=tuple)

    @property
    def weight_bytes(self) -> int:
        return sum(weight_bytes(j.fmt, j.n_out, self.n_in) for j in self.jobs)

    @property
    def flops(self) -> int:
        return sum(2 * self.t * j.n_out * self.n_in for j in self.jobs)


def _c4(t):
    # x rows are drawn in order, so every t sees the same first rows
    return Submission(f"c4_t{t}", 4, t, 5120, 0, 128, (Job(Q4, 17408, 1), Job(Q4, 17408, 2)))


SUBMISSIONS = {
    s.name: s
    for s in [
        # 1: one bf16 job, t = 1
        Submission("c1", 1, 1, 256, 0, 1, (Job(BF16, 1024, 1),)),
        # 2: fused bf16 decode, q/k/v-like, t = 1, one submission
        Submission("c2", 2, 1, 4096, 0, 1,
                   (Job(BF16, 4096, 1), Job(BF16, 1024, 2), Job(BF16, 1024, 3))),
        # 3: Q8 decode: gate + up on one x, then down on its own x
        Submission("c3a", 3, 1, 4096, 0, 1, (Job(Q8, 14336, 1), Job(Q8, 14336, 2))),
        Submission("c3b", 3, 1, 14336, 99, 1, (Job(Q8, 4096, 3),)),
        # 4: Q4 small-batch verify at t = 1, 2, 4, 8 (x rows are shared across t),
        # and at t = 16, 32, 64, 128 (mid-size verify batches)
        _c4(1), _c4(2), _c4(4), _c4(8), _c4(16), _c4(32), _c4(64), _c4(128),
        # 5: prefill: two bf16 jobs at t = 2048, a Q4 job on the first 512 rows
        Submission("c5a", 5, 2048, 4096, 0, 2048, (Job(BF16, 4096, 1), Job(BF16, 14336, 2))),
        Submission("c5b", 5, 512, 4096, 0, 2048, (Job(Q4, 14336, 3),)),
    ]
}


def make_x(sub: Submission) -> np.ndarray:
    return np.ascontiguousarray(gen_x(sub.cfg, sub.x_id, sub.x_rows, sub.n_in)[: sub.t])


def make_weights(sub: Submission) -> list:
    return [gen_weight(j.fmt, sub.cfg, j.tensor_id, j.n_out, sub.n_in) for j in sub.jobs]
