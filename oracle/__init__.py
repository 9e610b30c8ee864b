"""CPU oracle of the FlashHead Lite DiT slice denoiser -- TEST INFRASTRUCTURE.

A plain, slow, float64 numpy statement of what the audio-conditioned DiT and
its 4-step flow-matching sampler compute. It exists to check the HIP library
and nothing else: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path never
calls it, and it shares no code with the HIP library (only the seeded data of
``synth`` serves both).

Every function cites the passage of the pages it follows. Where the pages are
silent the plain reading taken is stated in the docstring as READING.

Pinning status: every function here is pinned by a CPU test against something
other than itself (library routines on special cases, closed forms,
invariants, brute force on tiny inputs); see ``tests/test_oracle_*.py``.
Agreement with a trained FlashHead checkpoint is "parity unpinned": no page
prints a tensor of the real model.
"""
from .dit import *  # noqa: F401,F403
from . import renoise  # noqa: F401
from . import mxfp8  # noqa: F401
from . import audio  # noqa: F401
from . import color  # noqa: F401
from . import vae  # noqa: F401
