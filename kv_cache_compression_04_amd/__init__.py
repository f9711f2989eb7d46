"""MI355X-native TurboQuant hot path: online KV encode, logits and attention
from packed codes.  The compute lives in libtq.so (include/tq.h); ``tq`` is
its Python binding and ``synth`` holds the seeded synthetic input recipes."""
from . import tq  # noqa: F401
