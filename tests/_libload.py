"""Helpers for tests: make sure libattn.so exists (build it once if nothing is built)."""
import os

import attention_attn_decode_amd as aa
from attention_attn_decode_amd import build as _build


def ensure_built():
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    return aa.lib()
