"""Shared test helpers: build-if-missing and loading of the library (no oracle arithmetic)."""
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_built():
    import token_sparse_attention_head_amd as tsa
    if not os.path.exists(tsa.LIB_PATH):
        from token_sparse_attention_head_amd import build
        build.build()
    return tsa
