"""Compressed token ids: the lookup table the hash reads first.

The walk-through (yaoyuxiang.cn/news/830577, section 2.2-1 and the
CompressedTokenizer of section 4.1) shrinks the vocabulary before hashing:
each token's text is normalised (Unicode NFKC, lower case, accents removed),
the normal form is the token's key (the text itself when the normal form is
empty), and tokens with equal keys share one compressed id.  The result is
the `remap` table of the engram parameters: remap[raw id] = compressed id.

Readings: the three named operations run in the order the page lists them;
"accents removed" drops the combining marks (Unicode category Mn) of the
canonical decomposition; "lower case" is str.lower (not case folding);
compressed ids are numbered by the first raw id (ascending) of each key; the
caller passes each token's decoded text (for byte-level vocabularies, the
text the token stands for).

Host code, run once per vocabulary.  Tokens made only of ASCII characters
(most of a BPE vocabulary) take a shortcut: for them NFKC and the
decomposition change nothing and no combining mark can occur, so the key is
the lower-cased text.
"""
from __future__ import annotations

import unicodedata
from typing import Iterable, Tuple

import numpy as np


def normalize(text: str) -> str:
    """NFKC, then lower case, then the combining marks of the canonical decomposition removed."""
    if text.isascii():
        return text.lower()
    t = unicodedata.normalize("NFKC", text).lower()
    return "".join(ch for ch in unicodedata.normalize("NFD", t) if unicodedata.category(ch) != "Mn")


def build_remap(texts: Iterable[str]) -> Tuple[np.ndarray, int]:
    """remap [V] int32 (raw id -> compressed id) and the compressed vocabulary size V'."""
    ids: dict = {}
    out = []
    for text in texts:
        norm = normalize(text)
        key = norm if norm else text
        cid = ids.get(key)
        if cid is None:
            cid = ids[key] = len(ids)
        out.append(cid)
    return np.asarray(out, dtype=np.int32), len(ids)
