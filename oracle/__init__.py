"""CPU oracle of the self-indexing compressed-key decode path (test infrastructure).

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it.  The product path (the HIP
library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path.

See ``oracle.sikv`` for the method, step by step.
"""

from .sikv import *  # noqa: F401,F403
