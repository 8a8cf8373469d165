"""The profile summaries' source stamp (CPU only): it covers the code of the
kernel sources, not their comments, and every committed profile matches the
sources in the tree, so bench.py reports the measured traffic."""

import glob
import os
import re

from yoco_shared_kv_gather_amd import profiling


def test_code_only_drops_comments_and_keeps_literals():
    text = 'int a = 1;  // note\n/* block\n   comment */ const char* s = "a//b /* c */";\nchar q = \'/\'; x = 2 / 2;\n'
    assert profiling.code_only(text) == 'int a = 1; const char* s = "a//b /* c */"; char q = \'/\'; x = 2 / 2;'
    # a comment edit leaves the code alone; a code edit does not
    assert profiling.code_only(text.replace("note", "another note")) == profiling.code_only(text)
    assert profiling.code_only(text.replace("x = 2", "x = 3")) != profiling.code_only(text)
    # an escaped quote inside a literal does not end it
    assert profiling.code_only('s = "a\\"//b"; // c') == 's = "a\\"//b";'


def test_committed_profiles_match_the_sources():
    paths = sorted(glob.glob(os.path.join(profiling.PROFILES, "*.md")))
    assert paths
    for path in paths:
        stem = os.path.basename(path)[:-3]
        m = re.search(r"^source_hash: (\S+)", open(path).read(), re.M)
        assert m, stem
        assert m.group(1) == profiling.source_hash(stem), f"{stem}: sources changed since it was profiled"
