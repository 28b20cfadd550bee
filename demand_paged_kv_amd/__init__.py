"""libgrowpage: the GrowPage capacity-boundary engine for AMD MI355X (gfx950).

The compute lives in the HIP library ``libgrowpage.so`` (C ABI in include/growpage.h);
``binding`` marshals arguments to it and ``engine`` owns the device buffers of a batch.
"""
from . import binding  # noqa: F401
from .binding import GrowPageError, Params, params, params_from  # noqa: F401
