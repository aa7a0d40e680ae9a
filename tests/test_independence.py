"""The oracle and the product path share no code and neither imports the other."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_routed_amd")
ORC = os.path.join(ROOT, "oracle")


def _sources(d, exts):
    for dp, _, fs in os.walk(d):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_product_never_references_oracle():
    for p in _sources(PKG, (".py", ".hip", ".cpp", ".h", ".hpp")):
        txt = open(p).read()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", txt, re.M), p
        assert "liboracle" not in txt, p
        assert "oracle.c" not in txt, p


def test_oracle_never_references_product():
    for p in _sources(ORC, (".py", ".c", ".h")):
        txt = open(p).read()
        assert not re.search(r"^\s*(import|from)\s+mixture_experts_routed_amd\b", txt, re.M), p
        assert "libmoe" not in txt, p
        assert "#include \"" not in txt, p  # no shared headers
