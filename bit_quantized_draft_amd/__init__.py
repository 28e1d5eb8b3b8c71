"""SubSpec substitute-draft hot path on MI355X (gfx950).

The HIP library libsubspec.so (built in-tree from csrc/ by build.py) does every step;
this package is its C ABI (include/subspec.h) seen from Python, with torch supplying
device memory and streams. Importing it does not need a GPU; calling into it does.
"""

from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
