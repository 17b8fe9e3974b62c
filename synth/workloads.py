"""Shapes of the synthetic workloads shared by the tests, the bench and the smoke check.

Each workload is a looped-transformer KV cache quantized along the loop axis
(LoopVQ, "LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers",
arXiv 2611.05304, abstract): one b-bit codebook index covers c channels of G
consecutive loop steps.  The first ``prefix`` and last ``recent`` tokens of
every sequence stay bf16 (airadar.tv summary of LoopVQ, section "Utilisation":
8 prefix and 64 recent tokens in the authors' serving launch).

This module holds sizes only: no random numbers and none of the method's
arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int          # L
    loops: int           # T
    loop_group: int      # G (consecutive loop steps sharing one index)
    q_heads: int         # Hq
    kv_heads: int        # Hkv
    head_dim: int        # d
    chans: int           # c (channels per sub-vector and loop step)
    index_bits: int      # b, codebook size K = 2**b
    batch: int           # B sequences
    context: int         # N cached tokens per sequence (includes the token being decoded)
    prefix: int = 8      # P bf16 prefix tokens
    recent: int = 64     # R bf16 recent tokens
    page_tokens: int = 64
    outlier_channels: int = 0   # key channels per (layer, kv-head) scaled by outlier_scale
    outlier_scale: float = 10.0
    rotate_keys: bool = False   # keys carry a seeded random orthogonal rotation of head_dim
    codebook_per_loop_group: bool = False
    encode_tokens: int = 0      # tokens bulk-encoded by the encode benchmark (0: none)
    wid: int = 0                # workload id mixed into every seed

    # ----- derived sizes -----
    @property
    def groups(self) -> int:            # d / c channel groups
        return self.head_dim // self.chans

    @property
    def sub_len(self) -> int:           # c * G elements per sub-vector
        return self.chans * self.loop_group

    @property
    def codewords(self) -> int:         # K
        return 1 << self.index_bits

    @property
    def loop_groups(self) -> int:       # J = T / G
        return self.loops // self.loop_group

    @property
    def cb_loop_groups(self) -> int:    # Jcb
        return self.loop_groups if self.codebook_per_loop_group else 1

    @property
    def n_vq(self) -> int:
        return max(0, self.context - self.prefix - self.recent)

    @property
    def queries_per_launch(self) -> int:
        return self.batch * self.q_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Tiny case: the oracle runs it in seconds; covers encode and decode.
TINY = Workload(name="tiny_d64_n512", layers=1, loops=4, loop_group=4, q_heads=1, kv_heads=1,
                head_dim=64, chans=4, index_bits=8, batch=1, context=512, wid=1)

# One layer of a 1.4B-class looped model: 16 heads, d=128, batch 32, 4K context,
# 4 outlier key channels at 10x per head.
LAYER_4K = Workload(name="layer16h_d128_b32_n4k", layers=1, loops=4, loop_group=4, q_heads=16,
                    kv_heads=16, head_dim=128, chans=4, index_bits=8, batch=32, context=4096,
                    outlier_channels=4, wid=2)

# Full stack at long context: 24 layers x 4 loop steps, batch 64, 32K context, 0.5 bit/elem.
STACK_32K = Workload(name="stack24x4_h16_d128_b64_n32k", layers=24, loops=4, loop_group=4,
                     q_heads=16, kv_heads=16, head_dim=128, chans=4, index_bits=8, batch=64,
                     context=32768, outlier_channels=4, wid=3)

# 0.25 bit/elem: 8 channels x 4 loops per index, rotated keys, batch 128, 16K context.
QUARTER_16K = Workload(name="stack24x4_c8_rot_b128_n16k", layers=24, loops=4, loop_group=4,
                       q_heads=16, kv_heads=16, head_dim=128, chans=8, index_bits=8, batch=128,
                       context=16384, outlier_channels=4, rotate_keys=True, wid=4)

# Deep recurrence: 4 shared layers unrolled 32 loop steps (8 loop groups), 32 heads;
# decode at batch 16, 8K context; the encode benchmark bulk-quantizes 65536 tokens.
DEEP_8K = Workload(name="deep4x32_h32_d128_b16_n8k", layers=4, loops=32, loop_group=4,
                   q_heads=32, kv_heads=32, head_dim=128, chans=4, index_bits=8, batch=16,
                   context=8192, outlier_channels=4, encode_tokens=65536, wid=5)

ALL = [TINY, LAYER_4K, STACK_32K, QUARTER_16K, DEEP_8K]
BY_NAME = {w.name: w for w in ALL}
