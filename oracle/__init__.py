"""Oracle for block-diffusion attention: TEST INFRASTRUCTURE ONLY.

Only the test suite, the build entry point's smoke check and the benchmark's
CPU-baseline leg may import this package. It holds two oracles: the
block-diffusion attention (bdattn_oracle) and the token-chunked linear
cross-entropy (lce_oracle). The GPU library does not import,
link or call it, and it imports nothing from the GPU library.

Every function here is pinned by a CPU test against something other than
itself (a hand-drawn mask fixture, closed forms at Q = 0, a library attention
routine, scalar brute force, finite differences, invariants of the method).
"""
from .bdattn_oracle import (BLOCK_CAUSAL, CLEAN, CORRUPTED, TOKEN_CAUSAL, Layout, Oracle,
                            clean_key_positions, corrupted_copies, documents, key_positions, key_tokens, layout, merge_partials, query_positions,
                            query_tokens, round_bf16, visible)
from .lce_oracle import LinearCE

__all__ = ["BLOCK_CAUSAL", "CLEAN", "CORRUPTED", "TOKEN_CAUSAL", "Layout", "Oracle",
           "clean_key_positions", "corrupted_copies", "documents",
           "key_positions", "key_tokens", "layout", "merge_partials", "query_positions",
           "query_tokens", "round_bf16", "visible", "LinearCE"]
