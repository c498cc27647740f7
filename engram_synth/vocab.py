"""A seeded synthetic tokenizer vocabulary (token texts in raw-id order) for
the compressed-id lookup.  No tokenizer vocabulary file is available, so this
stands in for one: every text is unique, most are lower-case ASCII words
with or without a leading space, and about a quarter are other spellings of
an earlier word (capitalised, upper case, fullwidth letters, a precomposed
or combining accent on a vowel, Greek capitals, halfwidth katakana), the kind
of near-duplicates the walk-through's compression merges (about 23% fewer
ids on its tokenizer).  A few tokens are lone combining marks.

This module draws random numbers and spells strings; it applies no
normalisation (the spellings are chosen from the character tables below).
"""
from __future__ import annotations

from typing import List

import numpy as np

from . import stream_z

STREAM_VOCAB = 13

_CONS = "bcdfghjklmnprstvwz"
_VOW = "aeiou"
_ACUTE = {"a": "á", "e": "é", "i": "í", "o": "ó", "u": "ú"}
_GRAVE = {"a": "à", "e": "è", "i": "ì", "o": "ò", "u": "ù"}
_GREEK_LOWER = [chr(c) for c in range(0x3B1, 0x3CA) if c != 0x3C2]
_KATAKANA = ["カ", "キ", "ク", "ケ", "コ", "サ", "シ", "ス", "セ", "ソ"]
_HALFWIDTH = {"カ": "ｶ", "キ": "ｷ", "ク": "ｸ", "ケ": "ｹ", "コ": "ｺ",
              "サ": "ｻ", "シ": "ｼ", "ス": "ｽ", "セ": "ｾ", "ソ": "ｿ"}
_MARKS = ["̀", "́", "̂", "̃", "̈", "̊", "̌", "̧"]


def _word(z: int) -> str:
    n = 1 + z % 4
    z //= 4
    out = []
    for _ in range(n):
        out.append(_CONS[z % len(_CONS)])
        z //= len(_CONS)
        out.append(_VOW[z % len(_VOW)])
        z //= len(_VOW)
        if z % 3 == 0:
            out.append(_CONS[(z // 3) % len(_CONS)])
        z //= 3
    return "".join(out)


def _base(z: int) -> str:
    kind = z % 20
    z //= 20
    if kind == 0:    # Greek
        return "".join(_GREEK_LOWER[(z >> (5 * i)) % len(_GREEK_LOWER)] for i in range(1 + z % 3))
    if kind == 1:    # katakana
        return "".join(_KATAKANA[(z >> (4 * i)) % len(_KATAKANA)] for i in range(1 + z % 3))
    if kind == 2:    # CJK ideographs
        return "".join(chr(0x4E00 + (z >> (14 * i)) % 0x5000) for i in range(1 + z % 2))
    w = _word(z >> 2)
    return " " + w if z % 2 else w


def _variant(base: str, z: int) -> str:
    core = base.lstrip(" ")
    lead = base[: len(base) - len(core)]
    if core and core[0] in _GREEK_LOWER:
        return lead + core.upper()
    if core and core[0] in _HALFWIDTH:
        return lead + "".join(_HALFWIDTH.get(ch, ch) for ch in core)
    if not core or not core.isascii():
        return base
    kind = z % 6
    z //= 6
    vowels = [i for i, ch in enumerate(core) if ch in _VOW]
    if kind == 0:
        core = core.capitalize()
    elif kind == 1:
        core = core.upper()
    elif kind == 2:
        core = "".join(chr(ord(ch) - 0x20 + 0xFF00) if ch.isalpha() else ch for ch in core)
    elif kind in (3, 4) and vowels:
        i = vowels[z % len(vowels)]
        table = _ACUTE if kind == 3 else _GRAVE
        core = core[:i] + table[core[i]] + core[i + 1:]
    elif vowels:
        i = vowels[z % len(vowels)]
        core = core[: i + 1] + "́" + core[i + 1:]
    else:
        core = core.upper()
    return lead + core


def synthetic_vocab(seed: int, vocab: int, variant_share: float = 0.19) -> List[str]:
    """`vocab` unique token texts in raw-id order."""
    out: List[str] = []
    seen = set()
    bases: List[str] = []
    counter = 0
    for mark in _MARKS[: min(len(_MARKS), vocab // 1000)]:
        out.append(mark)
        seen.add(mark)
    cut = int(variant_share * 2**32)
    zs: List[int] = []
    while len(out) < vocab:
        if counter % 65536 == 0:
            zs = [int(x) for x in stream_z(seed, STREAM_VOCAB, np.arange(counter, counter + 65536, dtype=np.int64))]
        z = zs[counter % 65536]
        counter += 1
        if bases and (z & 0xFFFFFFFF) < cut:
            text = _variant(bases[(z >> 32) % len(bases)], z >> 45)
        else:
            text = _base(z >> 32)
            if text not in seen:
                bases.append(text)
        if text in seen:
            continue
        seen.add(text)
        out.append(text)
    return out
