"""MI355X (gfx950) sparse mixture-of-experts layer forward: C-ABI HIP library + ctypes binding."""
from . import moe  # noqa: F401
