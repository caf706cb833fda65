"""The five workload shapes (attention layer geometry + sharing topology).

Index 0 is the tiny fp32 case small enough for pure-Python brute force.
Indices 1-3 are decode workloads; index 4 is the chunked-prefill workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    dtype: str               # "f32" or "bf16" (storage and I/O element type)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rank: int
    lora_scale: float
    rope_theta: float
    sessions: int            # independent shared prefixes
    agents_per_session: int
    prefix_len: int          # shared-prefix tokens per session
    suffix_len: int          # private tokens each agent appends after the fork (decode)
    chunk_len: int           # prefill chunk per agent (0 for decode workloads)
    num_bpages: int
    num_rpages: int
    b_std: float             # std of the LoRA up-projections B_k, B_v
    page_size: int = 16
    kind: str = "decode"     # "decode" or "prefill"
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def n_agents(self) -> int:
        return self.sessions * self.agents_per_session

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def kv_width(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def seq_len(self) -> int:
        """Cached keys per agent at the decode call (prefix + private suffix)."""
        return self.prefix_len + self.suffix_len


def _pool_pages(needed: int) -> int:
    """Next power of two at or above 1.25x the pages a workload needs."""
    want = (needed * 5 + 3) // 4
    p = 1
    while p < want:
        p *= 2
    return p


def _decode_cfg(name, dtype, hq, hkv, d, r, s, theta, sessions, aps, prefix, suffix, b_std,
                seed, nb=None, nr=None, notes=""):
    P = 16
    need_b = sessions * (-(-prefix // P)) + sessions * aps * (-(-suffix // P))
    need_r = sessions * aps * (-(-(prefix + suffix) // P))
    return WorkloadConfig(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                          rank=r, lora_scale=s, rope_theta=theta, sessions=sessions,
                          agents_per_session=aps, prefix_len=prefix, suffix_len=suffix,
                          chunk_len=0, num_bpages=nb or _pool_pages(need_b),
                          num_rpages=nr or _pool_pages(need_r), b_std=b_std, seed=seed,
                          notes=notes)


CONFIGS = [
    _decode_cfg("tiny_f32", "f32", 4, 1, 64, 8, 2.0, 1e4, 1, 2, 64, 16, 0.05, seed=0,
                nb=32, nr=32, notes="2 agents, 64-token shared prefix, 16 private tokens each"),
    _decode_cfg("llama3_8b_react_decode", "bf16", 32, 8, 128, 16, 2.0, 5e5, 1, 4, 8192, 512,
                0.02, seed=1, notes="4 agents share 8192 tokens, 512 private each"),
    _decode_cfg("llama3_8b_mapreduce_decode", "bf16", 32, 8, 128, 16, 2.0, 5e5, 1, 8, 32768,
                1024, 0.02, seed=2, notes="8 agents share 32768 tokens, 1024 private each"),
    _decode_cfg("qwen25_14b_batched_decode", "bf16", 40, 8, 128, 16, 2.0, 1e6, 4, 8, 65536,
                2048, 0.02, seed=3, notes="4 sessions x 8 agents, 65536 shared + 2048 private"),
    WorkloadConfig(name="qwen3_8b_chunked_prefill", dtype="bf16", num_q_heads=32,
                   num_kv_heads=8, head_dim=128, rank=16, lora_scale=2.0, rope_theta=1e6,
                   sessions=1, agents_per_session=8, prefix_len=131072, suffix_len=0,
                   chunk_len=512, num_bpages=_pool_pages(131072 // 16 + 8 * 512 // 16),
                   num_rpages=_pool_pages(8 * (131072 + 512) // 16), b_std=0.02,
                   kind="prefill", seed=4,
                   notes="8 agents share 131072 tokens; each appends a 512-token chunk"),
]


def config_by_name(name: str) -> WorkloadConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
