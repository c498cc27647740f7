"""Compressed token ids, the ORACLE (test infrastructure only: the tests and
the smoke check use it; the product never imports it).

Written from the Engram walk-through (yaoyuxiang.cn/news/830577): section
2.2-1 normalises token text (NFKC, lower case, accents removed) so that
tokens with the same normal form share an id, and the CompressedTokenizer of
section 4.1 keys each token by its normal form, or by its text when the
normal form is empty.  The steps run one character class at a time, in the
page's order, with Python's unicodedata as the Unicode library.
"""
import unicodedata


def normal_form(text):
    """NFKC, then lower case, then accents removed (combining marks, category
    Mn, of the canonical decomposition)."""
    nfkc = unicodedata.normalize("NFKC", text)
    lowered = nfkc.lower()
    decomposed = unicodedata.normalize("NFD", lowered)
    kept = []
    for ch in decomposed:
        if unicodedata.category(ch) != "Mn":
            kept.append(ch)
    return "".join(kept)


def compressed_ids(texts):
    """[compressed id of raw id 0, 1, ...] and the number of distinct keys;
    ids are numbered by the first raw id that has each key."""
    first_id_of_key = {}
    remap = []
    for text in texts:
        norm = normal_form(text)
        if norm:
            key = norm
        else:
            key = text
        if key not in first_id_of_key:
            first_id_of_key[key] = len(first_id_of_key)
        remap.append(first_id_of_key[key])
    return remap, len(first_id_of_key)
