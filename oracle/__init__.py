"""Float64 CPU oracle for score-guided KV selection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``attention_score_guided_amd``) never imports it and shares no code with it.
"""
from .kvsel_oracle import *  # noqa: F401,F403
